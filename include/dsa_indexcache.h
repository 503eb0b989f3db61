/*
 * dsa_indexcache.h - C ABI of the MI355X (gfx950) IndexCache / DeepSeek
 * Sparse Attention hot path.
 *
 * Method: "IndexCache: Accelerating Sparse Attention via Cross-Layer Index
 * Reuse" (gist.science es/pt/it/de editions of the paper summary).
 *  - DSA layer (technical summary §1 on every edition): a lightning indexer
 *    scores every previous token for each query, a per-row top-k keeps the k
 *    most relevant positions, and core attention runs over those k only.
 *  - IndexCache (technical summary §2, "Arquitectura del Método" on the es
 *    edition, "Arquitetura" on pt): a binary pattern splits the layers into
 *    Full (F) layers, which run indexer + top-k and store the index set, and
 *    Shared (S) layers, which skip both and reuse the set of the nearest
 *    preceding F layer - one conditional branch in the inference loop.
 *
 * Conventions shared by every entry point
 *  - All pointers except `pattern`, `layers`, `shape`, `stats`, the size
 *    outputs and the arguments of the host-only search helpers are DEVICE
 *    pointers, 16-byte aligned, rows contiguous.  The
 *    caller owns every buffer; the library never allocates, frees or
 *    synchronises.  Work is enqueued on `stream` (0 = the null stream) and is
 *    complete when the caller synchronises that stream.
 *  - Query row t of sequence b sits at absolute position
 *    pos(b,t) = ctx_len[b] - T + t and sees keys 0..pos (causal).  Callers
 *    must keep T <= ctx_len[b] <= Lmax; the kernels clamp out-of-range values
 *    instead of faulting, the results of such rows are unspecified.
 *  - Arguments are validated on the host before anything is launched.  A
 *    failing check returns a non-zero status, launches nothing and leaves a
 *    message for dsa_last_error().  A failed launch returns DSA_ERR_HIP.
 *  - Calls are re-entrant across host threads and streams as long as each
 *    in-flight call has its own outputs and workspace.  The only global state
 *    is the per-thread error message.
 */
#ifndef DSA_INDEXCACHE_H
#define DSA_INDEXCACHE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, bad pattern */
  DSA_ERR_UNSUPPORTED = 2, /* a shape / dtype combination with no kernel     */
  DSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required     */
  DSA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed      */
} dsa_status_t;

typedef enum dsa_dtype {
  DSA_BF16 = 0,     /* bfloat16                                              */
  DSA_FP8_E4M3 = 1  /* OCP fp8 e4m3 ("fn") codes with one fp32 scale per row */
} dsa_dtype_t;

/* Message describing the last non-OK status returned on this host thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
const char* dsa_last_error(void);

/* Library version string, e.g. "0.1.0 gfx950". */
const char* dsa_version(void);

/*
 * Lightning-indexer scores (technical summary §1: the indexer scores all
 * previous tokens of every query; the form used is the DSA one)
 *
 *   scores[b,t,s] = sum_h w[b,t,h] * ReLU( q[b,t,h,:] . k[b,s,:] )  for s <= pos(b,t)
 *   scores[b,t,s] = -inf                                            for pos(b,t) < s < Lmax
 *
 * q        [B,T,H,D] `dtype` elements.
 * q_scale  [B,T,H] fp32 per-row dequantisation scale (> 0) if dtype is
 *          DSA_FP8_E4M3 (real q = code * scale), must be NULL for DSA_BF16.
 * w        [B,T,H] fp32 head weights, any sign (applied after the ReLU).
 * k        [B,Lmax,D] `dtype` elements (the indexer key cache).
 * k_scale  [B,Lmax] fp32 per-row scale (> 0) for fp8, NULL for bf16.
 * ctx_len  [B] int32 (device).
 * scores   [B,T,ld_scores] fp32 output; columns 0..Lmax-1 are written.
 * Supported: D in {64,128}, 1 <= H <= 64, Lmax * D * element size < 2^31,
 * ld_scores >= Lmax and a multiple of 4.  Products are exact in fp32 and
 * accumulate in fp32.
 */
dsa_status_t dsa_indexer_scores(const void* q, dsa_dtype_t dtype, const float* q_scale,
                                const float* w, const void* k, const float* k_scale,
                                const int32_t* ctx_len, int B, int T, int H, int D, int Lmax,
                                float* scores, int64_t ld_scores, hipStream_t stream);

/*
 * Per-row top-k (technical summary §1: keep the k most relevant tokens).
 * For each row the k visible positions (0..pos(b,t)) with the highest score
 * are written in ASCENDING position order; equal scores are broken toward
 * the lower position; rows with fewer than k visible positions are padded
 * with -1.  Scores are compared as fp32 values (-0 == +0); NaN is not
 * allowed.
 * scores [B,T,ld_scores] fp32 (only columns 0..pos(b,t) are read),
 * idx    [B,T,k] int32 output.  1 <= k <= 16384, ld_scores multiple of 4.
 * workspace: dsa_topk_workspace_size bytes (may be 0 / NULL when 0).  Few
 * long rows are split across workgroups that meet in a per-row histogram
 * kept in the workspace: the workspace must be zero-filled before its first
 * use, and every call leaves the part that must start at zero (its leading
 * histograms) zero again.
 */
dsa_status_t dsa_topk_workspace_size(int B, int T, int Lmax, int k, size_t* bytes);
dsa_status_t dsa_topk(const float* scores, int64_t ld_scores, const int32_t* ctx_len, int B,
                      int T, int Lmax, int k, int32_t* idx, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * Indexer scores and top-k in one pass (technical summary §1: the indexer
 * scores every previous token and keeps the k most relevant; the scores are
 * consumed only by that selection).  idx [B,T,k_sel] is exactly what
 * dsa_indexer_scores followed by dsa_topk write for the same inputs (the
 * same fp32 scores decide the same selection), but the scores never reach
 * memory.  Arguments are those of dsa_indexer_scores and dsa_topk (k_sel is
 * dsa_topk's k), with the same limits.
 *   One query row per sequence (decode): each workgroup keeps its keys'
 *   scores in LDS and compacts its own candidates against a lower bound of
 *   the row's threshold (the row histogram in the workspace as it stands;
 *   no workgroup waits for another), then one workgroup per row completes
 *   the selection from the finished histogram.  A row may split into at
 *   most 1024 workgroups (Lmax up to 8388608 fp8 keys at D = 128);
 *   dsa_indexer_topk_workspace_size returns DSA_ERR_UNSUPPORTED beyond.
 *   Workspace: zero-filled before its first use; every call leaves its
 *   leading histograms zero again (dsa_topk's layout, so one zero-filled
 *   buffer of the larger size serves both).
 *   Several query rows per sequence (prefill, the shapes the prefill
 *   indexer takes): each wave scores one row over all its keys and appends
 *   the scores at or above its running bound (the threshold bin of the keys
 *   seen so far) to the row's candidate list, then one workgroup per row
 *   selects among the candidates.  Workspace: 8 bytes per key and row plus
 *   4 per row; no state kept between calls.
 * Calls sharing a workspace must not run concurrently.
 */
dsa_status_t dsa_indexer_topk_workspace_size(int B, int T, int H, int D, dsa_dtype_t dtype,
                                             int Lmax, int k_sel, size_t* bytes);
dsa_status_t dsa_indexer_topk(const void* q, dsa_dtype_t dtype, const float* q_scale,
                              const float* w, const void* k, const float* k_scale,
                              const int32_t* ctx_len, int B, int T, int H, int D, int Lmax,
                              int k_sel, int32_t* idx, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Sparse MLA attention over the selected latent rows (technical summary §1:
 * core attention restricted to the k selected tokens, O(Lk)).  Absorbed MLA:
 * one latent row of d_qk values per token is shared by all Hq heads; logits
 * use all d_qk columns, values the first d_v columns:
 *
 *   logit_j = scale * q[b,t,h,:] . kv[b, idx[b,t,j], :]   for valid j
 *   out[b,t,h,:] = sum_j softmax(logit)_j * kv[b, idx[b,t,j], 0:d_v]
 *   lse[b,t,h]   = log(sum_j exp(logit_j))                 (natural log)
 *
 * An entry j is valid when 0 <= idx[b,t,j] <= pos(b,t); others (the -1
 * padding) are skipped.  A row with no valid entry gives out = 0, lse = -inf.
 * q [B,T,Hq,d_qk] bf16, kv [B,Lmax,d_qk] bf16, idx [B,T,k] int32,
 * out [B,T,Hq,d_v] bf16 (round to nearest even from fp32),
 * lse [B,T,Hq] fp32 or NULL.  Softmax and accumulation are fp32.
 * Supported: d_qk == 576, d_v == 512, Hq a multiple of 16 in 16..1024,
 * 1 <= k <= 65536, Lmax * d_qk * 2 < 2^31 (one sequence's latent rows).
 * workspace: dsa_sparse_attn_workspace_size bytes (may be 0 / NULL when
 * 0): when the selected rows are split across workgroups it holds the
 * per-slice outputs (bf16, normalised by their own softmax sums) and their
 * fp32 log-sum-exp until a combine pass merges them.
 */
dsa_status_t dsa_sparse_attn_workspace_size(int B, int T, int Hq, int k, int d_v,
                                            size_t* bytes);
dsa_status_t dsa_sparse_attn(const void* q, const void* kv, const int32_t* idx,
                             const int32_t* ctx_len, int B, int T, int Hq, int Lmax, int k,
                             int d_qk, int d_v, float scale, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * KV-cache append: the step that precedes the indexer and the attention in
 * every decode step and prefill chunk.  During autoregressive generation each
 * new token's key/value entries are added to the cache before it is attended
 * over (enigmasecurity.cl article on IndexCache, section "Fundamentos de la
 * Atención Dispersa en Transformadores"); under DSA a token brings two rows,
 * its latent MLA row and its lightning-indexer key (technical summary §1).
 *
 *   row t of sequence b goes to position p = ctx_len[b] - T + t, i.e. ctx_len
 *   already counts the T new tokens (the convention of every entry point).
 *   kv_cache[b,p,:] = bf16_rne(kv_new[b,t,:])
 *   k_cache[b,p,:]  = bf16_rne(k_new[b,t,:])                    (DSA_BF16)
 *   k_scale[b,p]    = amax / 448 (1 for an all-zero row), fp32   (DSA_FP8_E4M3)
 *   k_cache[b,p,:]  = e4m3fn_rne(k_new[b,t,:] / k_scale[b,p])   (fp32 division)
 * The fp8 form is the one dsa_indexer_scores reads: one scale per key row (a
 * 128-element block when D = 128).  Rounding is to nearest, ties to even;
 * a quotient of magnitude >= 464 (reachable only through non-finite or
 * out-of-range inputs) saturates to 448 instead of becoming NaN.
 *
 * kv_new   [B,T,d_qk] fp32, kv_cache [B,Lmax,d_qk] bf16 (in/out);
 * k_new    [B,T,D] fp32,    k_cache  [B,Lmax,D] `k_dtype` (in/out),
 * k_scale  [B,Lmax] fp32 (in/out) for DSA_FP8_E4M3, NULL for DSA_BF16.
 * ctx_len  [B] int32 (device).
 * Either pair may be skipped: kv_new and kv_cache both NULL (d_qk ignored)
 * appends indexer keys only; k_new, k_cache and k_scale all NULL (D and
 * k_dtype ignored) appends latent rows only; at least one pair is given.
 * Only the T rows of each sequence are written; a row whose p falls outside
 * 0..Lmax-1 is not written at all.  The new rows must not overlap the caches.
 * Supported: d_qk and D multiples of 4, 4 <= d_qk <= 4096, 4 <= D <= 256,
 * inputs finite.
 */
dsa_status_t dsa_kv_append(const float* kv_new, const float* k_new, const int32_t* ctx_len,
                           int B, int T, int Lmax, int d_qk, int D, dsa_dtype_t k_dtype,
                           void* kv_cache, void* k_cache, float* k_scale, hipStream_t stream);

/* Streaming-read probe: a measurement aid, not a step of the method.  For
 * benchmarks that compare the decode indexer's key sweep with a plain read of
 * the same number of bytes, i.e. the practical HBM ceiling of that sweep.
 * Reads `bytes` bytes of device memory at `src` once and keeps nothing:
 *   DSA_PROBE_TILES  - the indexer's own load pattern: `workgroups`
 *                      workgroups of eight waves, each owning a contiguous
 *                      run of 8 KB tiles that its waves take interleaved,
 *                      two tiles (16 KB) in flight per wave;
 *   DSA_PROBE_STRIDE - a grid-stride sweep by `workgroups` workgroups of
 *                      512 threads, eight 16-byte loads in flight per lane.
 * All loads are 16-byte non-temporal loads.  The loaded words are folded by
 * XOR and a lane writes its fold to *sink only when it equals one fixed
 * 32-bit value, so *sink (device int32, caller-owned) is almost never
 * written and its contents mean nothing.
 * src: device, 16-byte aligned, `bytes` a positive multiple of 8192;
 * workgroups in 1..65536; in the tiles form each workgroup's run must stay
 * below 2^31 bytes.  Violations return DSA_ERR_INVALID_ARG or
 * DSA_ERR_UNSUPPORTED before any launch.
 */
#define DSA_PROBE_TILES 0
#define DSA_PROBE_STRIDE 1
dsa_status_t dsa_probe_stream_read(const void* src, int64_t bytes, int workgroups, int form,
                                   int32_t* sink, hipStream_t stream);

/* One layer's device tensors for indexcache_run_stack.  q_idx / w / k_idx
 * (and the fp8 scales) are read on F layers only; q / kv / out (and lse)
 * only when shape->Hq > 0. */
typedef struct dsa_layer {
  const void* q_idx;         /* [B,T,H,D]        */
  const float* q_idx_scale;  /* [B,T,H] or NULL  */
  const float* w;            /* [B,T,H]          */
  const void* k_idx;         /* [B,Lmax,D]       */
  const float* k_idx_scale;  /* [B,Lmax] or NULL */
  const void* q;             /* [B,T,Hq,d_qk]    */
  const void* kv;            /* [B,Lmax,d_qk]    */
  void* out;                 /* [B,T,Hq,d_v]     */
  float* lse;                /* [B,T,Hq] or NULL */
} dsa_layer_t;

/* dsa_stack_shape_t.flags */
#define DSA_STACK_UNFUSED_TOPK 1 /* F layers: scores through score_buf, then top-k */

typedef struct dsa_stack_shape {
  int B, T, H, D, Lmax, k;
  int Hq, d_qk, d_v;       /* Hq == 0: indexer + top-k only, no attention */
  dsa_dtype_t idx_dtype;
  float scale;             /* softmax scale of the sparse attention       */
  int flags;               /* 0 or DSA_STACK_UNFUSED_TOPK                 */
} dsa_stack_shape_t;

typedef struct dsa_stack_stats {
  int n_indexer_calls;     /* == number of 'F' in the pattern */
  int n_topk_calls;
  int n_attn_calls;
} dsa_stack_stats_t;

/*
 * The IndexCache layer loop (technical summary §2).  pattern is a host
 * string of n_layers characters, each 'F' or 'S', starting with 'F' (an S
 * layer inherits from the nearest PRECEDING F layer, so a leading S has
 * nothing to inherit and is rejected).  For layer l:
 *   'F': scores = dsa_indexer_scores(layer l) into score_buf, then
 *        dsa_topk into idx_buf              (the index cache is written);
 *        for decode shapes that dsa_indexer_topk takes, unless flags holds
 *        DSA_STACK_UNFUSED_TOPK, dsa_indexer_topk into idx_buf instead
 *        (the same set; score_buf is then neither written nor needed and
 *        may be NULL; see indexcache_stack_fuses_topk)
 *   'S': nothing                            (idx_buf is reused in place)
 *   then, if Hq > 0, dsa_sparse_attn(layer l, idx_buf).
 * idx_buf [B,T,k] int32 holds the last F layer's set when the call returns.
 * score_buf [B,T,ld_scores] fp32 scratch, workspace sized by
 * indexcache_stack_workspace_size; like the top-k workspace it must be
 * zero-filled before its first use, and every call leaves the part that
 * must start at zero zero again.  Zero-initialise the shape (flags).
 * stats (host, may be NULL) receives the
 * number of kernels of each kind that were enqueued.
 */
dsa_status_t indexcache_stack_workspace_size(const dsa_stack_shape_t* shape, size_t* bytes);
/* *fused = 1 when indexcache_run_stack runs F layers of this shape through
 * dsa_indexer_topk (decode shapes it takes, flags without
 * DSA_STACK_UNFUSED_TOPK; score_buf may then be NULL), else 0. */
dsa_status_t indexcache_stack_fuses_topk(const dsa_stack_shape_t* shape, int* fused);
dsa_status_t indexcache_run_stack(const char* pattern, int n_layers, const dsa_layer_t* layers,
                                  const dsa_stack_shape_t* shape, const int32_t* ctx_len,
                                  int32_t* idx_buf, float* score_buf, int64_t ld_scores,
                                  void* workspace, size_t workspace_bytes,
                                  dsa_stack_stats_t* stats, hipStream_t stream);

/*
 * indexcache_run_stack without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, validation, kernels and
 * results as indexcache_run_stack; the workspace is instead a static device
 * array inside the library of DSA_NOALLOC_SCRATCH_BYTES bytes, which each GPU
 * the library runs on holds from the module's load until the process ends.
 * The call allocates and frees nothing.  A shape whose
 * indexcache_stack_workspace_size exceeds DSA_NOALLOC_SCRATCH_BYTES is
 * rejected with DSA_ERR_WORKSPACE before anything is launched (the decode
 * workloads need at most about 33 MiB: batch 64 x 32K context, 128 heads).
 * The scratch belongs to the device current at the call (the stream's
 * device); it keeps the previous call's contents, and each call first clears
 * the part that must start at zero with a small fill kernel on `stream` (no
 * memset node, so the call can be captured).  Calls that overlap on one GPU
 * (other threads or streams, no ordering between them) share that scratch
 * and race; order them on one stream.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dsa_status_t indexcache_run_stack_noalloc(const char* pattern, int n_layers,
                                          const dsa_layer_t* layers,
                                          const dsa_stack_shape_t* shape,
                                          const int32_t* ctx_len, int32_t* idx_buf,
                                          float* score_buf, int64_t ld_scores,
                                          dsa_stack_stats_t* stats, hipStream_t stream);

/*
 * Training-free pattern search (technical summary §2, part A of the two
 * configuration approaches: start from all-F and convert, one layer at a
 * time, the layer whose switch to S raises the calibration loss least).
 * Without a trained model the loss is a PROXY, built from a cost matrix:
 *
 *   cost[l*n + j], j < l: what layer l loses by attending with layer j's
 *   index set T_j instead of its own T_l (T = top-k of the layer's indexer);
 *     DSA_PROXY_OUTPUT: sum (o_l[T_j] - o_l[T_l])^2 / sum o_l[T_l]^2 over
 *       layer l's bf16 attention outputs (0/0 = 0, x/0 = +inf);
 *     DSA_PROXY_MISS:   1 - sum_rows |T_j ∩ T_l| / sum_rows |T_l|
 *       (0 when no row selects anything);
 *   cost[l*n + j] = 0 for j >= l.
 *   The cost of a pattern is sum over l, in layer order, of cost[l*n + src(l)]
 *   with src(l) the nearest F layer at or before l.
 */
typedef enum dsa_reuse_proxy {
  DSA_PROXY_OUTPUT = 0,
  DSA_PROXY_MISS = 1
} dsa_reuse_proxy_t;

/*
 * Cost matrix of a layer stack on the device.  Every layer is scored as an F
 * layer (indexer inputs are read on all layers).  cost: DEVICE [n_layers *
 * n_layers] fp64, row-major, fully written.  score_buf / ld_scores as for
 * indexcache_run_stack.  DSA_PROXY_OUTPUT needs shape->Hq > 0 and every
 * layer's q, kv and out: on return layers[l].out (and lse when non-NULL)
 * holds layer l's attention output over its own set, i.e. the all-F output.
 * DSA_PROXY_MISS reads no attention inputs (Hq is ignored).  k <= 8192.  The workspace
 * (indexcache_reuse_costs_workspace_size bytes) holds the n_layers index sets
 * and the reduction scratch; like the stack's, it must be zero-filled before
 * its first use and is left that way.  Work: n_layers indexer + top-k runs,
 * plus n_layers*(n_layers+1)/2 sparse attention runs for DSA_PROXY_OUTPUT.
 */
dsa_status_t indexcache_reuse_costs_workspace_size(const dsa_stack_shape_t* shape, int n_layers,
                                                   dsa_reuse_proxy_t proxy, size_t* bytes);
dsa_status_t indexcache_reuse_costs(int n_layers, const dsa_layer_t* layers,
                                    const dsa_stack_shape_t* shape, const int32_t* ctx_len,
                                    dsa_reuse_proxy_t proxy, double* cost, float* score_buf,
                                    int64_t ld_scores, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * Host-only helpers over a HOST copy of the cost matrix (entries finite or
 * +inf; NaN is rejected).  Both run on the calling thread and touch no GPU.
 *
 * indexcache_pattern_cost: the proxy loss of one pattern (validated like
 * indexcache_run_stack's).
 *
 * indexcache_greedy_search: starting from all-F, each of n_shared steps
 * (0 <= n_shared < n_layers) tries every F layer but layer 0 as S and keeps
 * the conversion with the lowest pattern cost, the lower layer on equal cost.
 * patterns: n_shared * (n_layers + 1) chars, row m receiving the
 * NUL-terminated pattern after step m + 1; totals: n_shared doubles, its cost.
 */
dsa_status_t indexcache_pattern_cost(const double* cost, int n_layers, const char* pattern,
                                     double* total);
dsa_status_t indexcache_greedy_search(const double* cost, int n_layers, int n_shared,
                                      char* patterns, double* totals);

#ifdef __cplusplus
}
#endif
#endif /* DSA_INDEXCACHE_H */
