/*
 * dsa.h - C ABI of the DeepSeek Sparse Attention (DSA) decode path for
 * AMD Instinct MI355X (gfx950).
 *
 * The path (DSA bullet of "MTP and sparse attention: NSA and DSA"):
 *   1. lightning indexer: for query row t and cached token s,
 *        I(t,s) = sum_h w(t,h) * ReLU(q(t,h) . k(s))
 *      over 64 heads of 128 dims, FP8 queries and keys with fp32 scales;
 *   2. top-k: each row keeps its k (= 2048) highest-scoring visible tokens;
 *   3. absorbed-form MLA over only those tokens: 128 heads score the
 *      576-wide bf16 latent (512 latent + 64 rope) and average its first 512
 *      dims, split over KV chunks with an online softmax and merged by
 *      log-sum-exp (stages 2 and 3 of the sparse decode in "Deepseek
 *      Details", section DSA).
 * Batches follow "[SGLang] NSA" (NSAMetadata, init_forward_metadata): a
 * request has 1 + MTP query rows, its cached length includes them, row j
 * of a request with n rows and L cached tokens sees the first L - n + 1 + j
 * tokens, and a page table maps positions to physical 64-token pages.
 *
 * Conventions for every entry point:
 *  - Pointers named in the argument lists are device pointers (HBM), owned
 *    by the caller, contiguous in the layouts stated; the library never
 *    allocates or frees on these calls and keeps no pointer after return.
 *  - Work is enqueued on the given HIP stream(s) (hipStream_t passed as
 *    void*; NULL = the null stream) and is asynchronous: no call waits for
 *    the device.  Calls on different streams that share a workspace race.
 *  - Host scalars are validated; device metadata (cu_seqlens_q, seqlens_k,
 *    page_table, idx) is trusted to be consistent with them, and kernels
 *    clamp it so a bad value never reads outside the buffers the host
 *    scalars describe.  A page id outside [0, num_pages) names no cached
 *    token: its positions score -inf in the indexer (below every real
 *    score, so a row selects them only when it has fewer than k keyed
 *    positions) and the attention skips them.
 *  - Every function returns a dsa_status; on error nothing is enqueued and
 *    dsa_last_error() returns a message (thread-local).  No exception or
 *    abort crosses the ABI.
 *  - bf16 values are passed as their 16-bit patterns (uint16_t); FP8 values
 *    are OCP e4m3fn codes (uint8_t).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_PAGE_SIZE 64  /* tokens per cache page */
#define DSA_IDX_HEADS 64  /* indexer heads */
#define DSA_IDX_DIM 128   /* indexer head dim (FP8) */
#define DSA_MLA_HEADS 128 /* MLA query heads */
#define DSA_MLA_DIM 576   /* latent + rope dims of a cached token */
#define DSA_MLA_DV 512    /* latent dims averaged into the output */
#define DSA_MAX_TOPK 8192 /* largest k accepted */

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent scalars */
  DSA_ERR_UNSUPPORTED = 2, /* a shape outside what the kernels implement */
  DSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than dsa_workspace_size() */
  DSA_ERR_HIP = 4,         /* a HIP launch or event call failed */
  DSA_ERR_DEVICE_CHECK = 5 /* checked builds: a kernel found bad device data
                            * (reported by dsa_device_check) */
} dsa_status;

/* One batch of requests (host struct; the arrays it points to are on the device).
 *  batch        B, number of requests (>= 0)
 *  num_tokens   T = cu_seqlens_q[B], total query rows
 *  max_q        >= every request's row count
 *  max_seqlen_k >= every seqlens_k[b]
 *  max_pages_per_req  row stride of page_table (>= ceil(max_seqlen_k / 64))
 *  num_pages    physical pages in the caches
 *  cu_seqlens_q int32 [B+1], cu[0] = 0, non-decreasing; rows of request b
 *               are cu[b] .. cu[b+1]-1
 *  seqlens_k    int32 [B], L_b: cached tokens of request b including its
 *               rows (L_b = 0 marks a padding request: no visible tokens)
 *  page_table   int32 [B, max_pages_per_req], physical page of logical page
 *               p of request b; entries past ceil(L_b/64) are never read */
typedef struct {
  int32_t batch;
  int32_t num_tokens;
  int32_t max_q;
  int32_t max_seqlen_k;
  int32_t max_pages_per_req;
  int32_t num_pages;
  const int32_t* cu_seqlens_q;
  const int32_t* seqlens_k;
  const int32_t* page_table;
} dsa_batch_t;

/* Lightning-indexer scores ("MTP and sparse attention: NSA and DSA", DSA
 * bullet; cache layout from the accounting listing: 128 FP8 bytes plus a
 * 4-byte scale per token).
 *  q8       uint8 [T, 64, 128]     indexer queries (e4m3fn)
 *  q_scale  f32 [T]                one positive scale per query row
 *  w        f32 [T, 64]            per-(row, head) weights (any sign)
 *  k8_cache uint8 [num_pages, 64, 128]  indexer keys by physical slot
 *  k_scale  f32 [num_pages, 64]    one positive scale per cached key
 *  scores   f32 [T, ld] out: scores[t, s] = q_scale[t] * k_scale[slot(s)] *
 *           sum_h w[t,h] * max(0, sum_d e4m3(q8[t,h,d]) * e4m3(k8[slot(s),d]))
 *           for s < v_t (row t's visible length), and -inf for the positions
 *           of a page whose id is outside [0, num_pages) (the pool holds no
 *           key for them); entries s >= v_t are not written.
 *           With positive scales this equals I(t,s) on the dequantised values.
 *  ld       >= max_seqlen_k
 * q8 and k8_cache must be 16-byte aligned, scores 4-byte.
 * Errors: INVALID_ARG (null pointers with T > 0, misalignment, ld too small,
 * bad scalars). */
int dsa_index_score(const dsa_batch_t* batch, const uint8_t* q8, const float* q_scale,
                    const float* w, const uint8_t* k8_cache, const float* k_scale, float* scores,
                    int64_t ld, void* stream);

/* Cache append: the step's new tokens into the two paged caches
 * ("MTP and sparse attention: NSA and DSA", new demands on inference
 * engines: the indexer keys form a second paged cache beside the latent, and
 * the cache accounting listing gives 128 FP8 bytes plus a 4-byte scale per
 * key; "[SGLang] NSA", forward_decode: the new tokens' latent rows are stored
 * into the paged pool before the attention runs).
 * Query row j of request b (n_b rows, L_b cached tokens including them) is
 * the token at position p = L_b - n_b + j; its slot is
 * page_table[b][p / 64] * 64 + p % 64.
 *  k_new    bf16 [T, 128]  the rows' indexer keys (finite values)
 *  kv_new   bf16 [T, 576]  the rows' latent (512) + rope (64) values
 *  k8_cache uint8 [num_pages, 64, 128] out: k8[slot, d] = e4m3fn(k_new[t, d] / s)
 *           rounded to nearest even, where s = max_d |k_new[t, d]| / 448 in
 *           fp32 (s = 1 for an all-zero key); the key's largest magnitude
 *           maps to +-448
 *  k_scale  f32 [num_pages, 64] out: k_scale[slot] = s
 *  kv_cache bf16 [num_pages, 64, 576] out: kv_cache[slot] = kv_new[t] (bit copy)
 * Slots of rows whose page id is outside [0, num_pages), or whose position
 * is negative, are not written; no other slot is touched.  kv_new and
 * kv_cache must be 16-byte aligned, k_new and k_scale 4-byte, k8_cache
 * 2-byte.
 * Errors: INVALID_ARG (null pointers with T > 0, misalignment, bad scalars). */
int dsa_cache_append(const dsa_batch_t* batch, const uint16_t* k_new, const uint16_t* kv_new,
                     uint8_t* k8_cache, float* k_scale, uint16_t* kv_cache, void* stream);

/* Per-row top-k over scores[t, 0 .. v_t) ("MTP and sparse attention: NSA
 * and DSA", DSA bullet: each query keeps its 2048 highest-scoring tokens).
 *  scores  f32 [T, ld]; -0.0 ranks as +0.0; NaN ranks above +inf
 *  k       1 .. DSA_MAX_TOPK
 *  idx     int32 [T, k] out: the K_t = min(k, v_t) selected logical positions
 *          (ties at the k-th score go to the lower position), stored in
 *          idx[t, 0 .. K_t) in ascending order, followed by -1 in
 *          idx[t, K_t .. k); the output is deterministic.
 *  ws      device workspace of >= dsa_workspace_size(DSA_OP_TOPK, ...) bytes,
 *          16-byte aligned
 * Errors: INVALID_ARG (also for a misaligned ws), WORKSPACE. */
int dsa_topk(const dsa_batch_t* batch, const float* scores, int64_t ld, int32_t k, int32_t* idx,
             void* ws, size_t ws_bytes, void* stream);

/* Index spaces for a selection ("[SGLang] NSA": the top-k's positions are
 * turned into page-table indices for the paged sparse kernel, or into
 * offsets of a ragged KV buffer, by a transform fused with the top-k). */
enum {
  DSA_IDX_LOGICAL = 0, /* positions within the request (0 .. v_t-1) */
  DSA_IDX_PAGED = 1,   /* physical slots: page_table[b][p / 64] * 64 + p % 64
                          (-1 where the page id is outside [0, num_pages)) */
  DSA_IDX_RAGGED = 2   /* kv_offsets[b] + p: a buffer holding each request's
                          tokens contiguously from kv_offsets[b] on */
};

/* Top-k fused with the transform of its output into an index space: the
 * selection of dsa_topk (same set, same ascending order of the positions
 * behind the entries), each entry reported in `space`; -1 padding as
 * dsa_topk.  kv_offsets: int32 [B], read for DSA_IDX_RAGGED only (the
 * caller keeps kv_offsets[b] + v_t within int32).
 * Errors: as dsa_topk, and INVALID_ARG for an unknown space or a NULL
 * kv_offsets with DSA_IDX_RAGGED. */
int dsa_topk_transform(const dsa_batch_t* batch, const float* scores, int64_t ld, int32_t k,
                       int32_t space, const int32_t* kv_offsets, int32_t* idx, void* ws,
                       size_t ws_bytes, void* stream);

/* Sparse absorbed-MLA decode over selected tokens ("MTP and sparse
 * attention: NSA and DSA", DSA bullet and per-pair cost; split-KV online
 * softmax + LSE merge per "Deepseek Details", DSA, stages 2-3).
 *  q        bf16 [T, 128, 576]       absorbed queries (512 latent + 64 rope)
 *  kv_cache bf16 [num_pages, 64, 576] latent cache by physical slot
 *  idx      int32 [T, k]             logical positions; entries < 0 or
 *           >= v_t are skipped (so -1 padding is allowed); positions must
 *           be distinct within a row
 *  sm_scale softmax scale on the 576-dim dot product (1/sqrt(192) for DSA)
 *  out      bf16 [T, 128, 512] out: softmax(sm_scale * q.kv) @ kv[:, :512],
 *           rounded to nearest even; zeros for a row with no valid entry
 *  lse      f32 [T, 128] out (may be NULL): natural-log sum of exp of the
 *           scaled scores (-inf for a row with no valid entry)
 *  n_split  KV splits per row (0 = choose), 1 .. 64
 *  ws       workspace (>= dsa_workspace_size(DSA_OP_SPARSE_MLA, ...))
 * q, kv_cache, out and ws must be 16-byte aligned.  q and the attended cache
 * rows must hold no NaN (the kernels are compiled on that assumption): with
 * one, out and lse are unspecified.
 * Errors: INVALID_ARG (also for misalignment), WORKSPACE. */
int dsa_sparse_mla_decode(const dsa_batch_t* batch, const uint16_t* q, const uint16_t* kv_cache,
                          const int32_t* idx, int32_t k, float sm_scale, uint16_t* out,
                          float* lse, int32_t n_split, void* ws, size_t ws_bytes, void* stream);

/* dsa_sparse_mla_decode over physical slots (DSA_IDX_PAGED, as
 * dsa_topk_transform writes them): slots int32 [T, k]; entries < 0 or
 * >= num_pages * 64 are skipped and the rest must be distinct within a row;
 * no page-table lookup is made (the batch's page table may be NULL when
 * max_seqlen_k is 0), and the caller vouches that the slots are the row's
 * selection.  Output and errors as dsa_sparse_mla_decode, whose workspace
 * size it shares. */
int dsa_sparse_mla_decode_paged(const dsa_batch_t* batch, const uint16_t* q,
                                const uint16_t* kv_cache, const int32_t* slots, int32_t k,
                                float sm_scale, uint16_t* out, float* lse, int32_t n_split,
                                void* ws, size_t ws_bytes, void* stream);

/* Dense absorbed-MLA decode: the attention of dsa_sparse_mla_decode over
 * every visible position 0 .. v_t-1 of each row, with no index array -- the
 * short-sequence fallback ("MTP and sparse attention: NSA and DSA": at short
 * contexts sparse attention saves little, and the DeepSeek-V3.2 report runs
 * short sequences densely).  With v_t <= k it equals dsa_sparse_mla_decode
 * over the top-k's selection, bit for bit (the top-k then selects every
 * position, in order); dsa_decode_step takes this form by itself when
 * max_seqlen_k <= k and skips the indexer scan.
 *  ws  >= dsa_workspace_size(DSA_OP_DENSE_MLA, batch, any k, n_split)
 * Errors: INVALID_ARG, WORKSPACE, UNSUPPORTED (max_seqlen_k > 131072). */
int dsa_dense_mla_decode(const dsa_batch_t* batch, const uint16_t* q, const uint16_t* kv_cache,
                         float sm_scale, uint16_t* out, float* lse, int32_t n_split, void* ws,
                         size_t ws_bytes, void* stream);

/* Masked multi-head attention in the expanded form, for short prefills
 * ("MTP and sparse attention: NSA and DSA", the caveat on short-sequence
 * prefill and the per-pair accounting beside the DSA table: dense prefill
 * attends in the expanded multi-head form at 2*H*(128+64) + 2*H*128 FLOPs
 * per pair, a third of the absorbed form's, and the DeepSeek-V3.2 report
 * emulates DSA's selection in it with a mask).  Per row t and head h, over
 * the positions the row attends -- those idx[t] lists (entries < 0 or >= v_t
 * are ignored), or every visible position 0 .. v_t-1 when idx is NULL --
 * leaving out positions on a page id outside the pool:
 *   z(s)     = sm_scale * (q_nope[t,h] . (W_UK[h] c(s)) + q_rope[t,h] . r(s))
 *   out[t,h] = sum_s softmax(z)(s) * (W_UV[h] c(s))
 *   lse[t,h] = ln sum_s e^z(s)
 * with c(s) the first 512 and r(s) the last 64 dims of position s's cached
 * row.  The library first writes W_UK[h] c(s) and W_UV[h] c(s) of every
 * cached position of each request into the workspace (bf16), then attends
 * over them in 64-position tiles.
 *  q_nope   bf16 [T, 128, 128]  query dims that meet the up-projected keys
 *  q_rope   bf16 [T, 128, 64]   query dims that meet the rope dims
 *  w_uk     bf16 [128, 128, 512] head h's key up-projection (row d: key dim d)
 *  w_uv     bf16 [128, 128, 512] head h's value up-projection
 *  kv_cache bf16 [num_pages, 64, 576] latent cache by physical slot
 *  idx      int32 [T, k] logical positions (distinct within a row), or NULL
 *  k        entries per idx row (1 .. 8192; ignored when idx is NULL)
 *  sm_scale softmax scale on the 192-dim dot product (1/sqrt(192) for DSA)
 *  out      bf16 [T, 128, 128] out: rounded to nearest even; zeros for a row
 *           that attends nothing
 *  lse      f32 [T, 128] out (may be NULL); -inf for a row that attends nothing
 *  ws       >= dsa_workspace_size(DSA_OP_MASKED_MHA, batch, k, 0) bytes:
 *           B * 128 * lp * 512 + B * lp * 128 + T * lp / 8 bytes, lp =
 *           max_seqlen_k rounded up to 64
 * Every pointer 16-byte aligned.  No input may hold a NaN (as for
 * dsa_sparse_mla_decode): with one, out and lse are unspecified.
 * Errors: INVALID_ARG, WORKSPACE, UNSUPPORTED (max_seqlen_k > 65536). */
int dsa_masked_mha_prefill(const dsa_batch_t* batch, const uint16_t* q_nope,
                           const uint16_t* q_rope, const uint16_t* w_uk, const uint16_t* w_uv,
                           const uint16_t* kv_cache, const int32_t* idx, int32_t k,
                           float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                           void* stream);

/* Indexer inputs of one layer (device pointers, layouts as dsa_index_score). */
typedef struct {
  const uint8_t* q8;
  const float* q_scale;
  const float* w;
  const uint8_t* k8_cache;
  const float* k_scale;
} dsa_indexer_inputs_t;

/* MLA inputs of one layer (layouts as dsa_sparse_mla_decode). */
typedef struct {
  const uint16_t* q;
  const uint16_t* kv_cache;
  float sm_scale;
} dsa_mla_inputs_t;

typedef enum {
  /* indexer -> top-k -> sparse MLA on the selection just made, on stream_main */
  DSA_MODE_FUSED = 0,
  /* Multi-layer Indexer ("Multi-layer Indexer: Overlapping Selection and
   * Attention in DeepSeek Sparse Attention", abstract): the attention reads
   * the previous indexer layer's selection (opts->attend_idx) on stream_main
   * while this call's indexer + top-k run concurrently on stream_aux and
   * write idx_out (the selection the next layer attends).  stream_main
   * waits for stream_aux before the call's work counts as done. */
  DSA_MODE_MLI = 1
} dsa_step_mode;
/* In MLI mode the aux stream's top-k writes idx_out while the main stream's
 * attention reads attend_idx, so the two ranges [ptr, ptr + T*k) must not
 * overlap (dsa_decode_step returns DSA_ERR_INVALID_ARG when they do). */

/* Stages of a step, in the order of the optional stage events. */
enum {
  DSA_STAGE_INDEX_SCORE = 0, /* the indexer scan kernel */
  DSA_STAGE_TOPK = 1,        /* top-k selection after the scan */
  DSA_STAGE_ATTENTION = 2,   /* sparse MLA and its split merge */
  DSA_NUM_STAGES = 3
};

typedef struct {
  int32_t mode;               /* dsa_step_mode */
  int32_t n_split;            /* as dsa_sparse_mla_decode (0 = choose; in
                               * MLI mode the choice keeps the attention to
                               * half the work-groups of the other modes, so
                               * the concurrent scan keeps CUs) */
  const int32_t* attend_idx;  /* MLI: int32 [T, k] selection the attention reads */
  /* Optional (NULL = none): 2 * DSA_NUM_STAGES caller-created hipEvent_t.
   * Event 2i is recorded just before stage i and event 2i+1 just after it,
   * on the stream that stage runs on, so hipEventElapsedTime over the pair
   * is that stage's device time.  The caller owns the events. */
  void* const* stage_events;
} dsa_step_opts_t;

/* One decode step of one layer: indexer scores, top-k, sparse MLA -- the
 * three parts of the DSA bullet of "MTP and sparse attention: NSA and DSA"
 * run back to back for a batch laid out as "[SGLang] NSA" describes it
 * (init_forward_metadata: 1 + MTP query rows per request, cached lengths
 * that include them, cumulative query offsets, a 64-token page table), with
 * the attention's KV splits merged by log-sum-exp as in "Deepseek Details",
 * section DSA, stages 2-3.  When max_seqlen_k <= k every row keeps all its
 * visible tokens, so the step writes that selection without scanning and
 * attends densely (same results as the scan would give).
 *  ix, mla   this layer's inputs
 *  k         tokens kept per row
 *  idx_out   int32 [T, k] out: the selection of ix (as dsa_topk)
 *  out, lse  as dsa_sparse_mla_decode; attention over idx_out (FUSED) or
 *            over opts->attend_idx (MLI)
 *  ws        >= dsa_workspace_size(DSA_OP_DECODE_STEP, ...) bytes
 *  stream_main, stream_aux  stream_aux is used only in MLI mode (must be
 *            non-NULL and differ from stream_main there)
 * mla->q, mla->kv_cache, out, ws, ix->q8 and ix->k8_cache must be 16-byte
 * aligned.
 * Errors: INVALID_ARG (also for misalignment), WORKSPACE, HIP. */
int dsa_decode_step(const dsa_batch_t* batch, const dsa_indexer_inputs_t* ix,
                    const dsa_mla_inputs_t* mla, int32_t k, const dsa_step_opts_t* opts,
                    int32_t* idx_out, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                    void* stream_main, void* stream_aux);

/* dsa_decode_step for callers that cannot allocate device memory: code
 * being captured into a HIP graph, tight serving loops, harnesses that
 * forbid allocation.  It takes no workspace: the step runs in a static
 * scratch array of 64 MiB that the library keeps in each device's memory
 * for the life of the process (the first call on a device resolves that
 * device's copy; make it outside graph capture).  It calls no allocator.
 * Arguments and results as dsa_decode_step, in FUSED mode only (opts->mode
 * must be DSA_MODE_FUSED; opts->n_split and opts->stage_events as there).
 * Every call on one device shares that device's scratch: calls that may
 * overlap on one device (different streams, different threads) race.  The
 * scratch keeps the last call's contents; the step clears what it needs
 * cleared itself.
 * Errors: as dsa_decode_step; WORKSPACE (nothing enqueued) when the batch's
 * step needs more than 64 MiB, i.e. more than
 * dsa_workspace_size(DSA_OP_DECODE_STEP, batch, k, n_split) allows. */
int dsa_decode_step_noalloc(const dsa_batch_t* batch, const dsa_indexer_inputs_t* ix,
                            const dsa_mla_inputs_t* mla, int32_t k, const dsa_step_opts_t* opts,
                            int32_t* idx_out, uint16_t* out, float* lse, void* stream);

/* One layer of a multi-layer decode (device pointers, layouts as above). */
typedef struct {
  dsa_indexer_inputs_t ix; /* read on the layers that keep an indexer only */
  dsa_mla_inputs_t mla;
  uint16_t* out;           /* bf16 [T, 128, 512] out */
  float* lse;              /* f32 [T, 128] out, or NULL */
} dsa_layer_t;

/* A stack of n_layers layers under a multi-layer indexer schedule ("Multi-
 * layer Indexer: Overlapping Selection and Attention in DeepSeek Sparse
 * Attention", abstract: IndexCache keeps the indexer on a fraction 1/r of
 * the layers and the others reuse the latest selection; MLI lets a layer
 * attend the previous indexer layer's selection so that its own indexer runs
 * concurrently with its attention; the two compose).
 * Layer l keeps an indexer iff l % retention == 0; its selection (as
 * dsa_topk) is written to sel[l / retention].  Layer l attends
 *   - with mli = 0: sel[l / retention] (on an indexer layer, its own, made
 *     first);
 *   - with mli = 1: sel[l / retention - 1] on an indexer layer l > 0 (its own
 *     indexer + top-k run meanwhile on stream_aux, as DSA_MODE_MLI), else
 *     sel[l / retention] (layer 0 selects first, then attends its own).
 * retention = 1 with mli = 0 is n_layers fused decode steps.
 *  layers   n_layers entries
 *  sel      int32 [ceil(n_layers / retention), T, k] out
 *  ws       >= dsa_workspace_size(DSA_OP_DECODE_STEP, batch, k, n_split)
 *  stream_aux  used when mli = 1 (non-NULL, different from stream_main)
 * Every pointer of every layer is checked (non-NULL, aligned as
 * dsa_decode_step asks) before anything is enqueued.
 * Errors: INVALID_ARG, WORKSPACE, UNSUPPORTED, HIP. */
int dsa_decode_layers(const dsa_batch_t* batch, int32_t n_layers, const dsa_layer_t* layers,
                      int32_t k, int32_t retention, int32_t mli, int32_t n_split, int32_t* sel,
                      void* ws, size_t ws_bytes, void* stream_main, void* stream_aux);

typedef enum {
  DSA_OP_TOPK = 1,
  DSA_OP_SPARSE_MLA = 2,
  DSA_OP_DECODE_STEP = 3,
  DSA_OP_DENSE_MLA = 4, /* k is not used */
  DSA_OP_MASKED_MHA = 5 /* k and n_split are not used */
} dsa_op;

/* Workspace bytes an op needs for this batch, k and n_split (0 = the
 * library's choice, as in the calls).  0 for an invalid request. */
size_t dsa_workspace_size(int op, const dsa_batch_t* batch, int32_t k, int32_t n_split);

/* KV splits the library chooses for a batch when n_split = 0 (the single
 * ops and FUSED steps; MLI steps choose at most this many). */
int32_t dsa_default_splits(const dsa_batch_t* batch, int32_t k);

/* Device checks.  The library is also built as libdsa_checked.so, compiled
 * with DSA_DEVICE_CHECKS: there its kernels test the device data they are
 * handed against the batch's host scalars and record what they find in a
 * device word (one per device, flags ORed by vector atomics), without
 * changing what they compute.  The page tables checked are those of
 * "[SGLang] NSA" (NSAMetadata); the index entries those the top-k hands the
 * sparse kernel.  Flags: */
#define DSA_CHECK_PAGE_ID 1u   /* a visible position (or a new token's slot)
                                  maps to a page id outside [0, num_pages) */
#define DSA_CHECK_INDEX 2u     /* an attention index entry below -1, at or past
                                  its row's visible length, or a slot outside
                                  the pool */
#define DSA_CHECK_NAN_SCORE 4u /* an indexer score, or a score given to the
                                  top-k, is NaN (normal builds rank NaN above
                                  +inf) */
#define DSA_CHECK_METADATA 8u  /* a request's cached length outside
                                  [0, max_seqlen_k], or its row count above
                                  max_q */
/* Reads and clears this device's check word.  Call it after the work to be
 * checked has finished (it synchronises `stream` itself before reading).
 * flags_out (may be NULL) receives the flags.  Returns DSA_ERR_DEVICE_CHECK
 * when any flag was set, DSA_OK otherwise; in normal builds the checks are
 * compiled out and it returns DSA_OK with 0.  Errors: HIP. */
int dsa_device_check(uint32_t* flags_out, void* stream);

/* 1 in libdsa_checked.so, 0 in libdsa.so. */
int32_t dsa_device_checks_enabled(void);

const char* dsa_status_string(int status);

/* Message of the last error on the calling thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
