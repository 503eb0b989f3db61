// Host-side launchers of the gfx950 kernels.  Shapes are validated by the
// C ABI layer before these are called; they only pick a launch
// configuration and enqueue work on the stream.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Indexer scores, one query row at a time, keys streamed from HBM (T == 1
// decode, and the row-wise fallback for prefill).  With row_hist non-null the
// kernel also adds, per row, the count of visible scores in each of the 4096
// bins of their top 12 order-preserving key bits (the first histogram of the
// top-k selection) into row_hist[row * 4096 + bin], which must start at zero.
hipError_t launch_indexer_decode(const void* q, bool fp8, const float* q_scale, const float* w,
                                 const void* k, const float* k_scale, const int32_t* ctx_len,
                                 int B, int T, int H, int D, int Lmax, float* scores,
                                 int64_t ld, uint32_t* row_hist, hipStream_t stream);

// Indexer scores for a prefill chunk (T > 1): MFMA tiles over (query, key).
hipError_t launch_indexer_prefill(const void* q, bool fp8, const float* q_scale, const float* w,
                                  const void* k, const float* k_scale, const int32_t* ctx_len,
                                  int B, int T, int H, int D, int Lmax, float* scores,
                                  int64_t ld, hipStream_t stream);
bool indexer_prefill_supported(int H, int D);

size_t topk_workspace_bytes(int B, int T, int Lmax, int k);
// The per-row histogram inside a top-k workspace, or null when this shape
// does not use one (rows selected by one workgroup each).
uint32_t* topk_row_hist(void* workspace, int B, int T, int Lmax, int k);
// hist_ready: the workspace's row histogram was already filled for these
// scores (by launch_indexer_decode), so the histogram pass is skipped.
hipError_t launch_topk(const float* scores, int64_t ld, const int32_t* ctx_len, int B, int T,
                       int Lmax, int k, int32_t* idx, void* workspace, size_t ws_bytes,
                       bool hist_ready, hipStream_t stream);

// Workspace of the chunked (few long rows) selection, in order: per-row
// 4096-bin histograms (zero before the first call, left zero by every call),
// per-row selection {b1, count above b1, listed}, per-chunk candidate counts,
// candidate keys and positions (Lmax per row; chunk c's slice starts at
// c * chunk).
constexpr int kTopkMaxChunks = 1024;
struct TopkWs {
  uint32_t* hist;
  uint32_t* sel;
  uint32_t* cnt;
  uint32_t* key;
  int32_t* pos;
};
size_t topk_chunk_ws_bytes(int rows, int Lmax, int n_chunks);
TopkWs topk_chunk_ws(void* ws, int rows, int Lmax, int n_chunks);
// Steps 3-4 of the selection from chunk slices already in w (one workgroup
// per row); scores may be null when no score row exists in memory.  With
// sel_from_hist the threshold bin is taken from the finished row histogram
// and the slices may hold extra entries below it; otherwise w.sel holds the
// row's selection and the slices exactly the keys in bins >= it.
hipError_t launch_topk_finish(const float* scores, int64_t ld, const int32_t* ctx_len, int B,
                              int T, int Lmax, int k, int chunk, int n_chunks, const TopkWs& w,
                              bool sel_from_hist, int32_t* idx, hipStream_t stream);

// Fused decode indexer + top-k: the indexer keeps each workgroup's scores in
// LDS, builds the selection's first histogram, compacts its own candidates
// against a lower bound of the threshold bin, and the finishing workgroup
// per row completes the selection.  Scores never reach memory.  Supported
// when the decode indexer runs (not the prefill kernel) and the plan fits
// (see indexer_topk_plan_ok); workspace as above.
bool indexer_topk_plan_ok(int B, int T, int D, bool fp8, int Lmax, int k);
size_t indexer_topk_workspace_bytes(int B, int T, int D, bool fp8, int Lmax, int k);
hipError_t launch_indexer_topk_decode(const void* q, bool fp8, const float* q_scale,
                                      const float* w, const void* k, const float* k_scale,
                                      const int32_t* ctx_len, int B, int T, int H, int D,
                                      int Lmax, int k_sel, int32_t* idx, void* workspace,
                                      hipStream_t stream);

// Prefill form of the fused indexer + top-k (T > 1, the prefill kernel's
// shapes): each wave scores one query row over all its keys and appends the
// scores in bins at or above its running bound to the row's candidate list;
// launch_topk_candidates then selects per row.  Workspace: candidate keys
// and positions (Lmax per row each), per-row counts; nothing to keep zero.
size_t indexer_topk_prefill_workspace_bytes(int B, int T, int Lmax);
hipError_t launch_indexer_topk_prefill(const void* q, bool fp8, const float* q_scale,
                                       const float* w, const void* k, const float* k_scale,
                                       const int32_t* ctx_len, int B, int T, int H, int D,
                                       int Lmax, int k_sel, int32_t* idx, void* workspace,
                                       hipStream_t stream);
// Per-row top-k among position-ordered candidate lists (key, position) of
// cnt[row] entries at row * Lmax, which hold every key of the row's top k.
hipError_t launch_topk_candidates(const int32_t* ctx_len, int B, int T, int Lmax, int k,
                                  const uint32_t* key, const int32_t* pos, const uint32_t* cnt,
                                  int32_t* idx, hipStream_t stream);

size_t sparse_attn_workspace_bytes(int B, int T, int Hq, int k, int d_v);
hipError_t launch_sparse_attn(const void* q, const void* kv, const int32_t* idx,
                              const int32_t* ctx_len, int B, int T, int Hq, int Lmax, int k,
                              float scale, void* out, float* lse, void* workspace,
                              size_t ws_bytes, hipStream_t stream);

// New token rows into the latent cache (bf16) and the indexer key cache (bf16,
// or fp8 with one fp32 scale per row).  A null kv_new / k_new skips that cache.
hipError_t launch_kv_append(const float* kv_new, const float* k_new, const int32_t* ctx_len,
                            int B, int T, int Lmax, int d_qk, int D, bool k_fp8, void* kv_cache,
                            void* k_cache, float* k_scale, hipStream_t stream);

// Streaming-read probe: reads tiles * 8192 bytes at src once (tiles form:
// the decode indexer's sweep over `workgroups` contiguous runs; stride form:
// a grid-stride sweep).  Writes *sink only on a one-in-2^32 fold value.
hipError_t launch_stream_probe(const void* src, int64_t tiles, int workgroups, bool stride_form,
                               int32_t* sink, hipStream_t stream);

// Pattern-search proxy costs.  Each writes one fp64 value to *dst (device)
// after a reduction whose per-workgroup partials go to `partials`, which
// must hold kReuseCostMaxGrid entries.
constexpr int kReuseCostMaxGrid = 1024;
hipError_t launch_fill_zero_f64(double* p, int64_t n, hipStream_t stream);
// sum (out - ref)^2 / sum ref^2 over `elems` bf16 values (elems % 8 == 0).
hipError_t launch_output_cost(const void* out, const void* ref, int64_t elems, double2* partials,
                              double* dst, hipStream_t stream);
// 1 - sum |reused ∩ own| / sum |own| over `rows` index lists of length
// k <= 8192 (a row is staged in LDS).
hipError_t launch_miss_cost(const int32_t* reused, const int32_t* own, int64_t rows, int k,
                            double2* partials, double* dst, hipStream_t stream);

}  // namespace dsa
