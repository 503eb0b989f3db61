// C ABI of the IndexCache / DSA hot path: host-side validation, dispatch to
// the gfx950 kernels and the F/S layer-stack driver.
//
// The layer loop follows the IndexCache paper summary (technical §2 on the
// gist.science es/pt/it/de editions): F layers run indexer + top-k and store
// the index set in the one index buffer, S layers run neither and attend with
// the buffer as the nearest preceding F layer left it.  The branch is taken
// on the host from the pattern string; nothing is copied for S layers.
#include "../../include/dsa_indexcache.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "launchers.hpp"

namespace {

thread_local std::string g_last_error;

dsa_status_t fail(dsa_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dsa_status_t ok() {
  g_last_error.clear();
  return DSA_OK;
}

dsa_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define CHECK_PTR(p)                                                                   \
  do {                                                                                 \
    if ((p) == nullptr) return fail(DSA_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);   \
    if (!aligned16(p))                                                                 \
      return fail(DSA_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, #p);      \
  } while (0)

#define CHECK(cond, st, ...)                          \
  do {                                                \
    if (!(cond)) return fail((st), __VA_ARGS__);      \
  } while (0)

constexpr int kMaxTopk = 16384;
constexpr int kMaxAttnK = 65536;
constexpr int kMaxSearchK = 8192;  // one row's index list is staged in 32 KB of LDS
// Kernels address one sequence's cache through a buffer resource with a
// 32-bit byte range.
constexpr int64_t kMaxSeqBytes = 2147483647LL;

dsa_status_t check_indexer(const char* fn, const void* q, dsa_dtype_t dtype,
                           const float* q_scale, const float* w, const void* k,
                           const float* k_scale, const int32_t* ctx_len, int B, int T, int H,
                           int D, int Lmax, const float* scores, int64_t ld,
                           bool with_scores = true) {
  CHECK(dtype == DSA_BF16 || dtype == DSA_FP8_E4M3, DSA_ERR_INVALID_ARG, "%s: unknown dtype %d",
        fn, (int)dtype);
  CHECK(B >= 1 && T >= 1 && Lmax >= 1, DSA_ERR_INVALID_ARG,
        "%s: need B, T, Lmax >= 1 (got %d, %d, %d)", fn, B, T, Lmax);
  CHECK(T <= Lmax, DSA_ERR_INVALID_ARG, "%s: T (%d) exceeds Lmax (%d)", fn, T, Lmax);
  CHECK((int64_t)B * T <= 65535, DSA_ERR_UNSUPPORTED, "%s: B*T (%lld) above 65535", fn,
        (long long)B * T);
  CHECK(D == 64 || D == 128, DSA_ERR_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", fn, D);
  CHECK(H >= 1 && H <= 64, DSA_ERR_UNSUPPORTED, "%s: H must be in 1..64 (got %d)", fn, H);
  CHECK((int64_t)Lmax * D * (dtype == DSA_BF16 ? 2 : 1) <= kMaxSeqBytes, DSA_ERR_UNSUPPORTED,
        "%s: one sequence's key cache (Lmax %d x D %d) exceeds %lld bytes", fn, Lmax, D,
        (long long)kMaxSeqBytes);
  if (with_scores)
    CHECK(ld >= Lmax && ld % 4 == 0, DSA_ERR_INVALID_ARG,
          "%s: ld_scores (%lld) must be >= Lmax (%d) and a multiple of 4", fn, (long long)ld,
          Lmax);
  CHECK_PTR(q);
  CHECK_PTR(w);
  CHECK_PTR(k);
  CHECK_PTR(ctx_len);
  if (with_scores) CHECK_PTR(scores);
  if (dtype == DSA_FP8_E4M3) {
    CHECK(q_scale != nullptr && k_scale != nullptr, DSA_ERR_INVALID_ARG,
          "%s: fp8 inputs need q_scale and k_scale", fn);
    CHECK_PTR(q_scale);
    CHECK_PTR(k_scale);
  } else {
    CHECK(q_scale == nullptr && k_scale == nullptr, DSA_ERR_INVALID_ARG,
          "%s: bf16 inputs take no scales", fn);
  }
  return DSA_OK;
}

dsa_status_t check_topk(const char* fn, const float* scores, int64_t ld, const int32_t* ctx_len,
                        int B, int T, int Lmax, int k, const int32_t* idx,
                        bool with_scores = true) {
  CHECK(B >= 1 && T >= 1 && Lmax >= 1, DSA_ERR_INVALID_ARG,
        "%s: need B, T, Lmax >= 1 (got %d, %d, %d)", fn, B, T, Lmax);
  CHECK(T <= Lmax, DSA_ERR_INVALID_ARG, "%s: T (%d) exceeds Lmax (%d)", fn, T, Lmax);
  CHECK(k >= 1, DSA_ERR_INVALID_ARG, "%s: k must be >= 1 (got %d)", fn, k);
  CHECK(k <= kMaxTopk, DSA_ERR_UNSUPPORTED, "%s: k (%d) above %d", fn, k, kMaxTopk);
  CHECK((int64_t)B * T <= 2147483647LL / 2, DSA_ERR_UNSUPPORTED, "%s: too many rows", fn);
  if (with_scores) {
    CHECK(ld >= Lmax && ld % 4 == 0, DSA_ERR_INVALID_ARG,
          "%s: ld_scores (%lld) must be >= Lmax (%d) and a multiple of 4", fn, (long long)ld,
          Lmax);
    CHECK_PTR(scores);
  }
  CHECK_PTR(ctx_len);
  CHECK_PTR(idx);
  return DSA_OK;
}

dsa_status_t check_attn(const char* fn, const void* q, const void* kv, const int32_t* idx,
                        const int32_t* ctx_len, int B, int T, int Hq, int Lmax, int k, int d_qk,
                        int d_v, float scale, const void* out, const float* lse) {
  CHECK(B >= 1 && T >= 1 && Lmax >= 1, DSA_ERR_INVALID_ARG,
        "%s: need B, T, Lmax >= 1 (got %d, %d, %d)", fn, B, T, Lmax);
  CHECK(T <= Lmax, DSA_ERR_INVALID_ARG, "%s: T (%d) exceeds Lmax (%d)", fn, T, Lmax);
  CHECK(d_qk == 576 && d_v == 512, DSA_ERR_UNSUPPORTED,
        "%s: only d_qk = 576, d_v = 512 is built (got %d, %d)", fn, d_qk, d_v);
  CHECK(Hq >= 16 && Hq % 16 == 0 && Hq <= 1024, DSA_ERR_UNSUPPORTED,
        "%s: Hq must be a multiple of 16 in 16..1024 (got %d)", fn, Hq);
  CHECK(k >= 1 && k <= kMaxAttnK, DSA_ERR_UNSUPPORTED, "%s: k must be in 1..%d (got %d)", fn,
        kMaxAttnK, k);
  CHECK((int64_t)Lmax * d_qk * 2 <= kMaxSeqBytes, DSA_ERR_UNSUPPORTED,
        "%s: Lmax (%d) latent rows of %d bf16 exceed %lld bytes per sequence", fn, Lmax, d_qk,
        (long long)kMaxSeqBytes);
  CHECK((int64_t)B * T <= 2147483647LL / 2, DSA_ERR_UNSUPPORTED, "%s: too many rows", fn);
  CHECK(scale > 0.f && scale == scale, DSA_ERR_INVALID_ARG, "%s: scale must be > 0", fn);
  CHECK_PTR(q);
  CHECK_PTR(kv);
  CHECK_PTR(idx);
  CHECK_PTR(ctx_len);
  CHECK_PTR(out);
  if (lse != nullptr) CHECK_PTR(lse);
  return DSA_OK;
}

// The stack's workspace holds the top-k region (which must stay zero between
// calls) followed by the attention region.
bool uses_prefill_indexer(int T, int H, int D) { return T > 1 && dsa::indexer_prefill_supported(H, D); }

// The fused indexer + top-k applies: every prefill shape of the prefill
// kernel, and decode shapes whose workgroup plan fits the finishing kernel.
bool fused_topk_applies(int B, int T, int H, int D, dsa_dtype_t dtype, int Lmax, int k) {
  return uses_prefill_indexer(T, H, D) ||
         dsa::indexer_topk_plan_ok(B, T, D, dtype == DSA_FP8_E4M3, Lmax, k);
}

size_t fused_topk_bytes(int B, int T, int H, int D, dsa_dtype_t dtype, int Lmax, int k) {
  return uses_prefill_indexer(T, H, D)
             ? dsa::indexer_topk_prefill_workspace_bytes(B, T, Lmax)
             : dsa::indexer_topk_workspace_bytes(B, T, D, dtype == DSA_FP8_E4M3, Lmax, k);
}

hipError_t launch_fused_topk(const void* q, dsa_dtype_t dtype, const float* q_scale,
                             const float* w, const void* k, const float* k_scale,
                             const int32_t* ctx_len, int B, int T, int H, int D, int Lmax,
                             int k_sel, int32_t* idx, void* workspace, hipStream_t stream) {
  const bool fp8 = dtype == DSA_FP8_E4M3;
  if (uses_prefill_indexer(T, H, D))
    return dsa::launch_indexer_topk_prefill(q, fp8, q_scale, w, k, k_scale, ctx_len, B, T, H, D,
                                            Lmax, k_sel, idx, workspace, stream);
  return dsa::launch_indexer_topk_decode(q, fp8, q_scale, w, k, k_scale, ctx_len, B, T, H, D,
                                         Lmax, k_sel, idx, workspace, stream);
}

// The stack fuses decode F layers only: for prefill chunks the fused form
// is slower than the separate kernels on the benchmark's scores (its running
// bound lists about a quarter of each row) and needs 8 bytes per key per row.
bool stack_fuses_topk(const dsa_stack_shape_t* s) {
  return !(s->flags & DSA_STACK_UNFUSED_TOPK) && !uses_prefill_indexer(s->T, s->H, s->D) &&
         fused_topk_applies(s->B, s->T, s->H, s->D, s->idx_dtype, s->Lmax, s->k);
}

// Room for the separate top-k's workspace and for the fused path's (both
// start with the same zero-kept histograms).
size_t topk_region(const dsa_stack_shape_t* s) {
  size_t b = dsa::topk_workspace_bytes(s->B, s->T, s->Lmax, s->k);
  if (!uses_prefill_indexer(s->T, s->H, s->D) &&
      fused_topk_applies(s->B, s->T, s->H, s->D, s->idx_dtype, s->Lmax, s->k))
    b = std::max(b, fused_topk_bytes(s->B, s->T, s->H, s->D, s->idx_dtype, s->Lmax, s->k));
  return (b + 255) & ~size_t(255);
}

// One 'F' or 'S' per layer, starting with 'F'.
dsa_status_t check_pattern(const char* fn, const char* pattern, int n_layers) {
  CHECK(pattern != nullptr, DSA_ERR_INVALID_ARG, "%s: pattern is NULL", fn);
  CHECK(n_layers >= 1, DSA_ERR_INVALID_ARG, "%s: n_layers must be >= 1", fn);
  const size_t plen = strnlen(pattern, (size_t)n_layers + 1);
  CHECK(plen == (size_t)n_layers, DSA_ERR_INVALID_ARG,
        "%s: pattern length %zu does not match n_layers %d", fn, plen, n_layers);
  for (int l = 0; l < n_layers; ++l)
    CHECK(pattern[l] == 'F' || pattern[l] == 'S', DSA_ERR_INVALID_ARG,
          "%s: pattern[%d] = '%c' is neither 'F' nor 'S'", fn, l, pattern[l]);
  CHECK(pattern[0] == 'F', DSA_ERR_INVALID_ARG,
        "%s: pattern must start with 'F' (an S layer reuses the nearest preceding F)", fn);
  return DSA_OK;
}

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Workspace of the cost-matrix builder, in order: the top-k region (kept
// zero between calls), the attention region, the n index sets, one
// attention output for the reused sets, the reduction partials.
struct ReuseLayout {
  size_t attn, attn_bytes, sets, tmp, partials, total;
};

ReuseLayout reuse_layout(const dsa_stack_shape_t* s, int n, bool output) {
  ReuseLayout L;
  size_t off = topk_region(s);
  L.attn = off;
  L.attn_bytes = output ? dsa::sparse_attn_workspace_bytes(s->B, s->T, s->Hq, s->k, s->d_v) : 0;
  off += align256(L.attn_bytes);
  L.sets = off;
  off += align256((size_t)n * s->B * s->T * s->k * sizeof(int32_t));
  L.tmp = off;
  if (output) off += align256((size_t)s->B * s->T * s->Hq * s->d_v * 2);
  L.partials = off;
  off += align256((size_t)dsa::kReuseCostMaxGrid * sizeof(double2));
  L.total = off;
  return L;
}

// Proxy loss of a validated pattern: sum over layers, in order, of
// C[l][src(l)], src(l) the nearest F layer at or before l.
double pattern_total(const double* C, int n, const char* p) {
  double t = 0.0;
  int src = 0;
  for (int l = 0; l < n; ++l) {
    if (p[l] == 'F') src = l;
    t += C[(size_t)l * n + src];
  }
  return t;
}

dsa_status_t check_cost_matrix(const char* fn, const double* C, int n) {
  CHECK(C != nullptr, DSA_ERR_INVALID_ARG, "%s: cost is NULL", fn);
  CHECK(n >= 1 && n <= 4096, DSA_ERR_INVALID_ARG, "%s: n_layers must be in 1..4096 (got %d)",
        fn, n);
  for (size_t i = 0; i < (size_t)n * n; ++i)
    CHECK(C[i] == C[i], DSA_ERR_INVALID_ARG, "%s: cost[%zu] is NaN", fn, i);
  return DSA_OK;
}

// row_hist: optional per-row top-k histogram filled on the way (decode kernel
// only; pass null otherwise).
dsa_status_t run_indexer(const void* q, dsa_dtype_t dtype, const float* q_scale, const float* w,
                         const void* k, const float* k_scale, const int32_t* ctx_len, int B,
                         int T, int H, int D, int Lmax, float* scores, int64_t ld,
                         uint32_t* row_hist, hipStream_t stream) {
  const bool fp8 = dtype == DSA_FP8_E4M3;
  hipError_t e;
  if (uses_prefill_indexer(T, H, D))
    e = dsa::launch_indexer_prefill(q, fp8, q_scale, w, k, k_scale, ctx_len, B, T, H, D, Lmax,
                                    scores, ld, stream);
  else
    e = dsa::launch_indexer_decode(q, fp8, q_scale, w, k, k_scale, ctx_len, B, T, H, D, Lmax,
                                   scores, ld, row_hist, stream);
  return hip_status(e, "indexer launch");
}

// Validation shared by both stack entry points: pattern, flags, every
// layer's pointers and sizes; *need receives the workspace bytes.  Nothing
// is launched.
dsa_status_t check_stack(const char* fn, const char* pattern, int n_layers,
                         const dsa_layer_t* layers, const dsa_stack_shape_t* shape,
                         const int32_t* ctx_len, int32_t* idx_buf, float* score_buf,
                         int64_t ld_scores, size_t* need) {
  CHECK(pattern != nullptr && layers != nullptr && shape != nullptr, DSA_ERR_INVALID_ARG,
        "%s: pattern, layers and shape must be non-NULL", fn);
  {
    dsa_status_t st = check_pattern(fn, pattern, n_layers);
    if (st != DSA_OK) return st;
  }
  const dsa_stack_shape_t& s = *shape;
  CHECK(s.Hq >= 0, DSA_ERR_INVALID_ARG, "%s: Hq must be >= 0", fn);
  CHECK((s.flags & ~DSA_STACK_UNFUSED_TOPK) == 0, DSA_ERR_INVALID_ARG, "%s: unknown flags 0x%x",
        fn, (unsigned)s.flags);
  const bool fused = stack_fuses_topk(shape);
  {
    dsa_status_t st = indexcache_stack_workspace_size(shape, need);
    if (st != DSA_OK) return st;
  }
  char what[96];
  for (int l = 0; l < n_layers; ++l) {
    const dsa_layer_t& L = layers[l];
    snprintf(what, sizeof(what), "%s (layer %d)", fn, l);
    if (pattern[l] == 'F') {
      dsa_status_t st = check_indexer(what, L.q_idx, s.idx_dtype, L.q_idx_scale, L.w, L.k_idx,
                                      L.k_idx_scale, ctx_len, s.B, s.T, s.H, s.D, s.Lmax,
                                      score_buf, ld_scores, !fused);
      if (st != DSA_OK) return st;
      st = check_topk(what, score_buf, ld_scores, ctx_len, s.B, s.T, s.Lmax, s.k, idx_buf,
                      !fused);
      if (st != DSA_OK) return st;
    }
    if (s.Hq > 0) {
      dsa_status_t st = check_attn(what, L.q, L.kv, idx_buf, ctx_len, s.B, s.T, s.Hq, s.Lmax,
                                   s.k, s.d_qk, s.d_v, s.scale, L.out, L.lse);
      if (st != DSA_OK) return st;
    }
  }
  return DSA_OK;
}

// The layer loop on a validated stack and a workspace of at least the
// stack's size: F layers write idx_buf, S layers reuse it, every layer
// attends when Hq > 0.
dsa_status_t launch_stack(const char* pattern, int n_layers, const dsa_layer_t* layers,
                          const dsa_stack_shape_t* shape, const int32_t* ctx_len,
                          int32_t* idx_buf, float* score_buf, int64_t ld_scores,
                          void* workspace, size_t workspace_bytes, dsa_stack_stats_t* stats,
                          hipStream_t stream) {
  const dsa_stack_shape_t& s = *shape;
  const bool fused = stack_fuses_topk(shape);
  const size_t tk_bytes = topk_region(shape);
  void* attn_ws = workspace ? static_cast<unsigned char*>(workspace) + tk_bytes : nullptr;
  dsa_stack_stats_t st_local = {0, 0, 0};
  // When the decode indexer runs and the top-k keeps a per-row histogram, the
  // indexer fills that histogram as it writes the scores and the top-k skips
  // its own histogram pass.
  uint32_t* row_hist = uses_prefill_indexer(s.T, s.H, s.D)
                           ? nullptr
                           : dsa::topk_row_hist(workspace, s.B, s.T, s.Lmax, s.k);
  for (int l = 0; l < n_layers; ++l) {
    const dsa_layer_t& L = layers[l];
    if (pattern[l] == 'F' && fused) {  // Full layer, scores kept on chip
      dsa_status_t st = hip_status(
          launch_fused_topk(L.q_idx, s.idx_dtype, L.q_idx_scale, L.w, L.k_idx, L.k_idx_scale,
                            ctx_len, s.B, s.T, s.H, s.D, s.Lmax, s.k, idx_buf, workspace,
                            stream),
          "fused indexer + top-k launch");
      if (st != DSA_OK) return st;
      st_local.n_indexer_calls++;
      st_local.n_topk_calls++;
    } else if (pattern[l] == 'F') {  // Full layer: fresh index set into the cache
      dsa_status_t st = run_indexer(L.q_idx, s.idx_dtype, L.q_idx_scale, L.w, L.k_idx,
                                    L.k_idx_scale, ctx_len, s.B, s.T, s.H, s.D, s.Lmax,
                                    score_buf, ld_scores, row_hist, stream);
      if (st != DSA_OK) return st;
      st_local.n_indexer_calls++;
      st = hip_status(dsa::launch_topk(score_buf, ld_scores, ctx_len, s.B, s.T, s.Lmax, s.k,
                                       idx_buf, workspace, tk_bytes, row_hist != nullptr,
                                       stream),
                      "topk launch");
      if (st != DSA_OK) return st;
      st_local.n_topk_calls++;
    }
    // Shared layer: idx_buf already holds the nearest preceding F layer's set.
    if (s.Hq > 0) {
      dsa_status_t st = hip_status(
          dsa::launch_sparse_attn(L.q, L.kv, idx_buf, ctx_len, s.B, s.T, s.Hq, s.Lmax, s.k,
                                  s.scale, L.out, L.lse, attn_ws, workspace_bytes - tk_bytes,
                                  stream),
          "sparse attention launch");
      if (st != DSA_OK) return st;
      st_local.n_attn_calls++;
    }
  }
  if (stats) *stats = st_local;
  return ok();
}

// ---- Static scratch of indexcache_run_stack_noalloc (for callers that
// cannot allocate).  Each GPU the library runs on holds its own copy of this
// array until the process ends; host code never passes the array's name to a
// kernel (on the host it is only a stand-in), but the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.
constexpr size_t kNoAllocScratchBytes = DSA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dsa_status_t scratch_for_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  CHECK(dev >= 0 && dev < kMaxDevices, DSA_ERR_UNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(DSA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

// Bytes at the start of a stack workspace that must be zero when a call
// starts: the per-row top-k histograms (4096 32-bit bins per query row).
size_t stack_zero_prefix(const dsa_stack_shape_t* s) {
  return (size_t)s->B * s->T * 4096 * sizeof(uint32_t);
}

__global__ void zero_fill_kernel(uint4* __restrict__ p, size_t n16) {
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = z;
}

// bytes: a multiple of 16 (workspace regions are 256-byte aligned).
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const unsigned grid = (unsigned)std::min<size_t>(1024, (n16 + 255) / 256);
  hipLaunchKernelGGL(zero_fill_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace

extern "C" {

const char* dsa_last_error(void) { return g_last_error.c_str(); }

const char* dsa_version(void) { return "0.1.0 gfx950"; }

dsa_status_t dsa_indexer_scores(const void* q, dsa_dtype_t dtype, const float* q_scale,
                                const float* w, const void* k, const float* k_scale,
                                const int32_t* ctx_len, int B, int T, int H, int D, int Lmax,
                                float* scores, int64_t ld_scores, hipStream_t stream) {
  const char* fn = "dsa_indexer_scores";
  dsa_status_t st = check_indexer(fn, q, dtype, q_scale, w, k, k_scale, ctx_len, B, T, H, D,
                                  Lmax, scores, ld_scores);
  if (st != DSA_OK) return st;
  return run_indexer(q, dtype, q_scale, w, k, k_scale, ctx_len, B, T, H, D, Lmax, scores,
                     ld_scores, nullptr, stream);
}

dsa_status_t dsa_topk_workspace_size(int B, int T, int Lmax, int k, size_t* bytes) {
  const char* fn = "dsa_topk_workspace_size";
  CHECK(bytes != nullptr, DSA_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  CHECK(B >= 1 && T >= 1 && Lmax >= 1 && k >= 1, DSA_ERR_INVALID_ARG, "%s: bad sizes", fn);
  *bytes = dsa::topk_workspace_bytes(B, T, Lmax, k);
  return ok();
}

dsa_status_t dsa_topk(const float* scores, int64_t ld_scores, const int32_t* ctx_len, int B,
                      int T, int Lmax, int k, int32_t* idx, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "dsa_topk";
  dsa_status_t st = check_topk(fn, scores, ld_scores, ctx_len, B, T, Lmax, k, idx);
  if (st != DSA_OK) return st;
  const size_t need = dsa::topk_workspace_bytes(B, T, Lmax, k);
  CHECK(workspace_bytes >= need && (need == 0 || workspace != nullptr), DSA_ERR_WORKSPACE,
        "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
  if (need) CHECK_PTR(workspace);
  return hip_status(dsa::launch_topk(scores, ld_scores, ctx_len, B, T, Lmax, k, idx, workspace,
                                     workspace_bytes, false, stream),
                    "topk launch");
}

dsa_status_t dsa_indexer_topk_workspace_size(int B, int T, int H, int D, dsa_dtype_t dtype,
                                             int Lmax, int k, size_t* bytes) {
  const char* fn = "dsa_indexer_topk_workspace_size";
  CHECK(bytes != nullptr, DSA_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  CHECK(B >= 1 && T >= 1 && Lmax >= 1 && k >= 1 && H >= 1 && (D == 64 || D == 128),
        DSA_ERR_INVALID_ARG, "%s: bad sizes", fn);
  CHECK(dtype == DSA_BF16 || dtype == DSA_FP8_E4M3, DSA_ERR_INVALID_ARG, "%s: unknown dtype %d",
        fn, (int)dtype);
  CHECK(fused_topk_applies(B, T, H, D, dtype, Lmax, k), DSA_ERR_UNSUPPORTED,
        "%s: no fused plan for B=%d T=%d H=%d D=%d Lmax=%d (a decode row split into more "
        "than %d workgroups: use dsa_indexer_scores + dsa_topk)",
        fn, B, T, H, D, Lmax, dsa::kTopkMaxChunks);
  *bytes = fused_topk_bytes(B, T, H, D, dtype, Lmax, k);
  return ok();
}

dsa_status_t dsa_indexer_topk(const void* q, dsa_dtype_t dtype, const float* q_scale,
                              const float* w, const void* k, const float* k_scale,
                              const int32_t* ctx_len, int B, int T, int H, int D, int Lmax,
                              int k_sel, int32_t* idx, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  const char* fn = "dsa_indexer_topk";
  dsa_status_t st = check_indexer(fn, q, dtype, q_scale, w, k, k_scale, ctx_len, B, T, H, D,
                                  Lmax, nullptr, 0, false);
  if (st != DSA_OK) return st;
  st = check_topk(fn, nullptr, 0, ctx_len, B, T, Lmax, k_sel, idx, false);
  if (st != DSA_OK) return st;
  size_t need = 0;
  st = dsa_indexer_topk_workspace_size(B, T, H, D, dtype, Lmax, k_sel, &need);
  if (st != DSA_OK) return st;
  CHECK(workspace_bytes >= need, DSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given",
        fn, need, workspace_bytes);
  CHECK_PTR(workspace);
  return hip_status(launch_fused_topk(q, dtype, q_scale, w, k, k_scale, ctx_len, B, T, H, D,
                                     Lmax, k_sel, idx, workspace, stream),
                    "fused indexer + top-k launch");
}

dsa_status_t dsa_sparse_attn_workspace_size(int B, int T, int Hq, int k, int d_v,
                                            size_t* bytes) {
  const char* fn = "dsa_sparse_attn_workspace_size";
  CHECK(bytes != nullptr, DSA_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
  CHECK(B >= 1 && T >= 1 && Hq >= 16 && Hq % 16 == 0 && k >= 1 && d_v == 512,
        DSA_ERR_INVALID_ARG, "%s: bad sizes", fn);
  *bytes = dsa::sparse_attn_workspace_bytes(B, T, Hq, k, d_v);
  return ok();
}

dsa_status_t dsa_sparse_attn(const void* q, const void* kv, const int32_t* idx,
                             const int32_t* ctx_len, int B, int T, int Hq, int Lmax, int k,
                             int d_qk, int d_v, float scale, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "dsa_sparse_attn";
  dsa_status_t st =
      check_attn(fn, q, kv, idx, ctx_len, B, T, Hq, Lmax, k, d_qk, d_v, scale, out, lse);
  if (st != DSA_OK) return st;
  const size_t need = dsa::sparse_attn_workspace_bytes(B, T, Hq, k, d_v);
  CHECK(workspace_bytes >= need && (need == 0 || workspace != nullptr), DSA_ERR_WORKSPACE,
        "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
  if (need) CHECK_PTR(workspace);
  return hip_status(dsa::launch_sparse_attn(q, kv, idx, ctx_len, B, T, Hq, Lmax, k, scale, out,
                                            lse, workspace, workspace_bytes, stream),
                    "sparse attention launch");
}

dsa_status_t dsa_kv_append(const float* kv_new, const float* k_new, const int32_t* ctx_len,
                           int B, int T, int Lmax, int d_qk, int D, dsa_dtype_t k_dtype,
                           void* kv_cache, void* k_cache, float* k_scale, hipStream_t stream) {
  const char* fn = "dsa_kv_append";
  CHECK(B >= 1 && T >= 1 && Lmax >= 1, DSA_ERR_INVALID_ARG,
        "%s: need B, T, Lmax >= 1 (got %d, %d, %d)", fn, B, T, Lmax);
  CHECK(T <= Lmax, DSA_ERR_INVALID_ARG, "%s: T (%d) exceeds Lmax (%d)", fn, T, Lmax);
  CHECK((kv_new == nullptr) == (kv_cache == nullptr), DSA_ERR_INVALID_ARG,
        "%s: kv_new and kv_cache must be given together", fn);
  CHECK((k_new == nullptr) == (k_cache == nullptr), DSA_ERR_INVALID_ARG,
        "%s: k_new and k_cache must be given together", fn);
  CHECK(kv_new != nullptr || k_new != nullptr, DSA_ERR_INVALID_ARG,
        "%s: nothing to append (both row pointers are NULL)", fn);
  CHECK_PTR(ctx_len);
  bool fp8 = false;
  if (kv_new != nullptr) {
    CHECK(d_qk >= 4 && d_qk <= 4096 && d_qk % 4 == 0, DSA_ERR_UNSUPPORTED,
          "%s: d_qk must be a multiple of 4 in 4..4096 (got %d)", fn, d_qk);
    CHECK_PTR(kv_new);
    CHECK_PTR(kv_cache);
  } else {
    d_qk = 0;
  }
  if (k_new != nullptr) {
    CHECK(k_dtype == DSA_BF16 || k_dtype == DSA_FP8_E4M3, DSA_ERR_INVALID_ARG,
          "%s: unknown dtype %d", fn, (int)k_dtype);
    CHECK(D >= 4 && D <= 256 && D % 4 == 0, DSA_ERR_UNSUPPORTED,
          "%s: D must be a multiple of 4 in 4..256 (got %d)", fn, D);
    CHECK_PTR(k_new);
    CHECK_PTR(k_cache);
    fp8 = k_dtype == DSA_FP8_E4M3;
    if (fp8) {
      CHECK(k_scale != nullptr, DSA_ERR_INVALID_ARG, "%s: an fp8 key cache needs k_scale", fn);
      CHECK_PTR(k_scale);
    } else {
      CHECK(k_scale == nullptr, DSA_ERR_INVALID_ARG, "%s: a bf16 key cache takes no k_scale",
            fn);
    }
  } else {
    CHECK(k_scale == nullptr, DSA_ERR_INVALID_ARG, "%s: k_scale given without k_new", fn);
    D = 0;
  }
  return hip_status(dsa::launch_kv_append(kv_new, k_new, ctx_len, B, T, Lmax, d_qk, D, fp8,
                                          kv_cache, k_cache, k_scale, stream),
                    "kv append launch");
}

dsa_status_t dsa_probe_stream_read(const void* src, int64_t bytes, int workgroups, int form,
                                   int32_t* sink, hipStream_t stream) {
  const char* fn = "dsa_probe_stream_read";
  CHECK_PTR(src);
  CHECK_PTR(sink);
  CHECK(bytes > 0 && bytes % 8192 == 0, DSA_ERR_INVALID_ARG,
        "%s: bytes must be a positive multiple of 8192 (got %lld)", fn, (long long)bytes);
  CHECK(workgroups >= 1 && workgroups <= 65536, DSA_ERR_INVALID_ARG,
        "%s: workgroups must be in 1..65536 (got %d)", fn, workgroups);
  CHECK(form == DSA_PROBE_TILES || form == DSA_PROBE_STRIDE, DSA_ERR_INVALID_ARG,
        "%s: unknown form %d", fn, form);
  const int64_t tiles = bytes / 8192;
  // Tiles form: each workgroup's run is addressed through one 32-bit buffer range.
  CHECK(form != DSA_PROBE_TILES || (tiles + workgroups - 1) / workgroups * 8192 <= kMaxSeqBytes,
        DSA_ERR_UNSUPPORTED, "%s: %lld bytes over %d workgroups exceeds 2^31 - 1 per workgroup",
        fn, (long long)bytes, workgroups);
  return hip_status(dsa::launch_stream_probe(src, tiles, workgroups, form == DSA_PROBE_STRIDE,
                                             sink, stream),
                    "stream probe launch");
}

dsa_status_t indexcache_stack_workspace_size(const dsa_stack_shape_t* s, size_t* bytes) {
  const char* fn = "indexcache_stack_workspace_size";
  CHECK(s != nullptr && bytes != nullptr, DSA_ERR_INVALID_ARG, "%s: NULL argument", fn);
  CHECK(s->B >= 1 && s->T >= 1 && s->Lmax >= 1 && s->k >= 1, DSA_ERR_INVALID_ARG,
        "%s: bad sizes", fn);
  size_t need = topk_region(s);
  if (s->Hq > 0) {
    CHECK(s->Hq % 16 == 0 && s->d_v == 512, DSA_ERR_INVALID_ARG, "%s: bad attention sizes", fn);
    need += dsa::sparse_attn_workspace_bytes(s->B, s->T, s->Hq, s->k, s->d_v);
  }
  *bytes = need;
  return ok();
}

dsa_status_t indexcache_stack_fuses_topk(const dsa_stack_shape_t* s, int* fused) {
  const char* fn = "indexcache_stack_fuses_topk";
  CHECK(s != nullptr && fused != nullptr, DSA_ERR_INVALID_ARG, "%s: NULL argument", fn);
  *fused = stack_fuses_topk(s) ? 1 : 0;
  return ok();
}

dsa_status_t indexcache_run_stack(const char* pattern, int n_layers, const dsa_layer_t* layers,
                                  const dsa_stack_shape_t* shape, const int32_t* ctx_len,
                                  int32_t* idx_buf, float* score_buf, int64_t ld_scores,
                                  void* workspace, size_t workspace_bytes,
                                  dsa_stack_stats_t* stats, hipStream_t stream) {
  const char* fn = "indexcache_run_stack";
  size_t need = 0;
  dsa_status_t st = check_stack(fn, pattern, n_layers, layers, shape, ctx_len, idx_buf,
                                score_buf, ld_scores, &need);
  if (st != DSA_OK) return st;
  CHECK(workspace_bytes >= need && (need == 0 || workspace != nullptr), DSA_ERR_WORKSPACE,
        "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
  if (stack_fuses_topk(shape) || need) CHECK_PTR(workspace);
  return launch_stack(pattern, n_layers, layers, shape, ctx_len, idx_buf, score_buf, ld_scores,
                      workspace, workspace_bytes, stats, stream);
}

dsa_status_t indexcache_run_stack_noalloc(const char* pattern, int n_layers,
                                          const dsa_layer_t* layers,
                                          const dsa_stack_shape_t* shape,
                                          const int32_t* ctx_len, int32_t* idx_buf,
                                          float* score_buf, int64_t ld_scores,
                                          dsa_stack_stats_t* stats, hipStream_t stream) {
  const char* fn = "indexcache_run_stack_noalloc";
  size_t need = 0;
  dsa_status_t st = check_stack(fn, pattern, n_layers, layers, shape, ctx_len, idx_buf,
                                score_buf, ld_scores, &need);
  if (st != DSA_OK) return st;
  CHECK(need <= kNoAllocScratchBytes, DSA_ERR_WORKSPACE,
        "%s: this shape needs %zu bytes of scratch; the library's static scratch holds %zu "
        "(use indexcache_run_stack with a workspace)",
        fn, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  st = scratch_for_current_device(fn, &ws);
  if (st != DSA_OK) return st;
  // The scratch keeps whatever the previous call on this GPU left in it: the
  // part that must start at zero (the top-k row histograms, at its start) is
  // cleared with a fill kernel, never a memset node, so that the call may be
  // captured into a graph.
  const size_t zero = std::min(topk_region(shape), stack_zero_prefix(shape));
  if (zero) {
    st = hip_status(launch_zero_fill(ws, zero, stream), "scratch clear launch");
    if (st != DSA_OK) return st;
  }
  return launch_stack(pattern, n_layers, layers, shape, ctx_len, idx_buf, score_buf, ld_scores,
                      ws, kNoAllocScratchBytes, stats, stream);
}

dsa_status_t indexcache_reuse_costs_workspace_size(const dsa_stack_shape_t* s, int n_layers,
                                                   dsa_reuse_proxy_t proxy, size_t* bytes) {
  const char* fn = "indexcache_reuse_costs_workspace_size";
  CHECK(s != nullptr && bytes != nullptr, DSA_ERR_INVALID_ARG, "%s: NULL argument", fn);
  CHECK(n_layers >= 1, DSA_ERR_INVALID_ARG, "%s: n_layers must be >= 1", fn);
  CHECK(proxy == DSA_PROXY_OUTPUT || proxy == DSA_PROXY_MISS, DSA_ERR_INVALID_ARG,
        "%s: unknown proxy %d", fn, (int)proxy);
  CHECK(s->B >= 1 && s->T >= 1 && s->Lmax >= 1 && s->k >= 1, DSA_ERR_INVALID_ARG,
        "%s: bad sizes", fn);
  CHECK(s->k <= kMaxSearchK, DSA_ERR_UNSUPPORTED, "%s: k (%d) above %d", fn, s->k, kMaxSearchK);
  if (proxy == DSA_PROXY_OUTPUT)
    CHECK(s->Hq >= 16 && s->Hq % 16 == 0 && s->d_v == 512, DSA_ERR_INVALID_ARG,
          "%s: the output proxy needs attention sizes (Hq a multiple of 16, d_v 512)", fn);
  *bytes = reuse_layout(s, n_layers, proxy == DSA_PROXY_OUTPUT).total;
  return ok();
}

dsa_status_t indexcache_reuse_costs(int n_layers, const dsa_layer_t* layers,
                                    const dsa_stack_shape_t* shape, const int32_t* ctx_len,
                                    dsa_reuse_proxy_t proxy, double* cost, float* score_buf,
                                    int64_t ld_scores, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  const char* fn = "indexcache_reuse_costs";
  CHECK(layers != nullptr && shape != nullptr, DSA_ERR_INVALID_ARG,
        "%s: layers and shape must be non-NULL", fn);
  size_t need = 0;
  {
    dsa_status_t st = indexcache_reuse_costs_workspace_size(shape, n_layers, proxy, &need);
    if (st != DSA_OK) return st;
  }
  CHECK(workspace_bytes >= need, DSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given",
        fn, need, workspace_bytes);
  CHECK_PTR(workspace);
  CHECK_PTR(cost);
  const dsa_stack_shape_t& s = *shape;
  const bool output = proxy == DSA_PROXY_OUTPUT;
  const ReuseLayout W = reuse_layout(shape, n_layers, output);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  int32_t* sets = reinterpret_cast<int32_t*>(ws + W.sets);
  char what[96];
  for (int l = 0; l < n_layers; ++l) {
    const dsa_layer_t& L = layers[l];
    snprintf(what, sizeof(what), "%s (layer %d)", fn, l);
    dsa_status_t st = check_indexer(what, L.q_idx, s.idx_dtype, L.q_idx_scale, L.w, L.k_idx,
                                    L.k_idx_scale, ctx_len, s.B, s.T, s.H, s.D, s.Lmax,
                                    score_buf, ld_scores);
    if (st != DSA_OK) return st;
    st = check_topk(what, score_buf, ld_scores, ctx_len, s.B, s.T, s.Lmax, s.k, sets);
    if (st != DSA_OK) return st;
    if (output) {
      st = check_attn(what, L.q, L.kv, sets, ctx_len, s.B, s.T, s.Hq, s.Lmax, s.k, s.d_qk, s.d_v,
                      s.scale, L.out, L.lse);
      if (st != DSA_OK) return st;
    }
  }
  const int64_t rows = (int64_t)s.B * s.T;
  const size_t set_elems = (size_t)rows * s.k;
  const int64_t out_elems = rows * s.Hq * s.d_v;
  const size_t tk_bytes = topk_region(shape);
  void* attn_ws = W.attn_bytes ? ws + W.attn : nullptr;
  void* tmp = ws + W.tmp;
  double2* partials = reinterpret_cast<double2*>(ws + W.partials);
  uint32_t* row_hist = uses_prefill_indexer(s.T, s.H, s.D)
                           ? nullptr
                           : dsa::topk_row_hist(workspace, s.B, s.T, s.Lmax, s.k);
  dsa_status_t st =
      hip_status(dsa::launch_fill_zero_f64(cost, (int64_t)n_layers * n_layers, stream),
                 "cost fill launch");
  if (st != DSA_OK) return st;
  // Every layer's own index set.
  for (int l = 0; l < n_layers; ++l) {
    const dsa_layer_t& L = layers[l];
    st = run_indexer(L.q_idx, s.idx_dtype, L.q_idx_scale, L.w, L.k_idx, L.k_idx_scale, ctx_len,
                     s.B, s.T, s.H, s.D, s.Lmax, score_buf, ld_scores, row_hist, stream);
    if (st != DSA_OK) return st;
    st = hip_status(dsa::launch_topk(score_buf, ld_scores, ctx_len, s.B, s.T, s.Lmax, s.k,
                                     sets + l * set_elems, workspace, tk_bytes,
                                     row_hist != nullptr, stream),
                    "topk launch");
    if (st != DSA_OK) return st;
  }
  for (int l = 0; l < n_layers; ++l) {
    const dsa_layer_t& L = layers[l];
    const int32_t* own = sets + l * set_elems;
    if (output) {
      st = hip_status(dsa::launch_sparse_attn(L.q, L.kv, own, ctx_len, s.B, s.T, s.Hq, s.Lmax,
                                              s.k, s.scale, L.out, L.lse, attn_ws, W.attn_bytes,
                                              stream),
                      "sparse attention launch");
      if (st != DSA_OK) return st;
    }
    for (int j = 0; j < l; ++j) {
      const int32_t* reused = sets + j * set_elems;
      double* dst = cost + (size_t)l * n_layers + j;
      if (output) {
        st = hip_status(dsa::launch_sparse_attn(L.q, L.kv, reused, ctx_len, s.B, s.T, s.Hq,
                                                s.Lmax, s.k, s.scale, tmp, nullptr, attn_ws,
                                                W.attn_bytes, stream),
                        "sparse attention launch");
        if (st != DSA_OK) return st;
        st = hip_status(dsa::launch_output_cost(tmp, L.out, out_elems, partials, dst, stream),
                        "output cost launch");
      } else {
        st = hip_status(dsa::launch_miss_cost(reused, own, rows, s.k, partials, dst, stream),
                        "miss cost launch");
      }
      if (st != DSA_OK) return st;
    }
  }
  return ok();
}

dsa_status_t indexcache_pattern_cost(const double* cost, int n_layers, const char* pattern,
                                     double* total) {
  const char* fn = "indexcache_pattern_cost";
  CHECK(total != nullptr, DSA_ERR_INVALID_ARG, "%s: total is NULL", fn);
  dsa_status_t st = check_cost_matrix(fn, cost, n_layers);
  if (st != DSA_OK) return st;
  st = check_pattern(fn, pattern, n_layers);
  if (st != DSA_OK) return st;
  *total = pattern_total(cost, n_layers, pattern);
  return ok();
}

dsa_status_t indexcache_greedy_search(const double* cost, int n_layers, int n_shared,
                                      char* patterns, double* totals) {
  const char* fn = "indexcache_greedy_search";
  dsa_status_t st = check_cost_matrix(fn, cost, n_layers);
  if (st != DSA_OK) return st;
  CHECK(n_shared >= 0 && n_shared < n_layers, DSA_ERR_INVALID_ARG,
        "%s: n_shared must be in 0..%d (got %d)", fn, n_layers - 1, n_shared);
  CHECK(n_shared == 0 || (patterns != nullptr && totals != nullptr), DSA_ERR_INVALID_ARG,
        "%s: patterns and totals must be non-NULL", fn);
  std::string p((size_t)n_layers, 'F');
  for (int m = 0; m < n_shared; ++m) {
    int best = -1;
    double best_cost = 0.0;
    for (int l = 1; l < n_layers; ++l) {
      if (p[l] != 'F') continue;
      p[l] = 'S';
      const double c = pattern_total(cost, n_layers, p.c_str());
      p[l] = 'F';
      if (best < 0 || c < best_cost) {
        best = l;
        best_cost = c;
      }
    }
    p[best] = 'S';
    memcpy(patterns + (size_t)m * (n_layers + 1), p.c_str(), (size_t)n_layers + 1);
    totals[m] = best_cost;
  }
  return ok();
}

}  // extern "C"
