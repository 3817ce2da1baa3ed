// C ABI of the DSA decode path: host-side validation, workspace carve-up and
// stream orchestration.  All arithmetic runs in the HIP kernels.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <mutex>
#include <string>

#include "dsa.h"
#include "internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  g_err = std::string(where) + ": " + hipGetErrorString(e);
  return DSA_ERR_HIP;
}

using dsa::align_up;
using dsa::BatchArgs;

// host scalars of the batch
int check_batch(const dsa_batch_t* b) {
  if (!b) return fail(DSA_ERR_INVALID_ARG, "batch is NULL");
  if (b->batch < 0 || b->num_tokens < 0 || b->max_q < 0 || b->max_seqlen_k < 0 ||
      b->max_pages_per_req < 0 || b->num_pages < 0)
    return fail(DSA_ERR_INVALID_ARG, "negative batch scalar");
  if (b->batch > 0 && (!b->cu_seqlens_q || !b->seqlens_k))
    return fail(DSA_ERR_INVALID_ARG, "cu_seqlens_q / seqlens_k is NULL");
  if (b->batch == 0 && b->num_tokens != 0)
    return fail(DSA_ERR_INVALID_ARG, "num_tokens > 0 with no requests");
  if (b->num_tokens > 0 && (b->max_q < 1 || b->max_q > b->num_tokens))
    return fail(DSA_ERR_INVALID_ARG, "max_q must be in [1, num_tokens]");
  if (b->max_seqlen_k > 0) {
    if (!b->page_table) return fail(DSA_ERR_INVALID_ARG, "page_table is NULL");
    if ((int64_t)b->max_pages_per_req * DSA_PAGE_SIZE < b->max_seqlen_k)
      return fail(DSA_ERR_INVALID_ARG, "max_pages_per_req * 64 < max_seqlen_k");
    if (b->num_pages < 1) return fail(DSA_ERR_INVALID_ARG, "num_pages < 1");
  }
  return DSA_OK;
}

int64_t step_ld(const dsa_batch_t* b) { return (int64_t)align_up((size_t)b->max_seqlen_k, 64); }

struct StepWs {
  size_t scores_off, topk_off, mla_off, total;
};

StepWs step_layout(const dsa_batch_t* b, int used_splits) {
  const BatchArgs a = dsa::batch_args(*b);
  StepWs w;
  size_t off = 0;
  w.scores_off = off;
  off = align_up(off + (size_t)b->num_tokens * (size_t)step_ld(b) * 4, 256);
  w.topk_off = off;
  off = align_up(off + dsa::topk_ws_layout(a).total, 256);
  w.mla_off = off;
  off = align_up(off + dsa::mla_ws_layout(a, used_splits).total, 256);
  w.total = off;
  return w;
}

// The attention reads q and gathers latent rows in 16-byte pieces, and the
// output and the workspace partials move in 16-byte pieces too.
bool misaligned16(const void* p) { return ((uintptr_t)p & 15) != 0; }
int check_mla_align(const void* q, const void* kv_cache, const void* out, const void* ws) {
  if (misaligned16(q) || misaligned16(kv_cache) || misaligned16(out) || misaligned16(ws))
    return fail(DSA_ERR_INVALID_ARG, "q, kv_cache, out and ws need 16-byte alignment");
  return DSA_OK;
}

// The scan reads queries and keys in 16-byte pieces and writes scores in
// 4-byte ones (16-byte ones where a row is aligned).
int check_index_align(const void* q8, const void* k8_cache, const float* scores) {
  if (misaligned16(q8) || misaligned16(k8_cache) || ((uintptr_t)scores & 3) != 0)
    return fail(DSA_ERR_INVALID_ARG, "q8 and k8_cache need 16-byte, scores 4-byte alignment");
  return DSA_OK;
}

int resolve_splits(const dsa_batch_t* b, int32_t k, int32_t n_split, int* used,
                   int wgs = dsa::kAttnWGs) {
  if (n_split < 0 || n_split > dsa::kMaxSplits)
    return fail(DSA_ERR_INVALID_ARG, "n_split must be in [0, 64]");
  const int ns = n_split == 0 ? dsa::default_splits(dsa::batch_args(*b), k, wgs) : n_split;
  *used = dsa::mla_splits_used(k, ns);
  return DSA_OK;
}

// two events per thread and device for the cross-stream joins of MLI mode
struct EventPair {
  int device = -1;
  hipEvent_t start = nullptr, done = nullptr;
};
thread_local EventPair g_events;

int get_events(hipEvent_t* start, hipEvent_t* done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (g_events.device != dev) {
    hipEvent_t a = nullptr, c = nullptr;
    e = hipEventCreateWithFlags(&a, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
    e = hipEventCreateWithFlags(&c, hipEventDisableTiming);
    if (e != hipSuccess) {
      (void)hipEventDestroy(a);
      return hip_fail(e, "hipEventCreateWithFlags");
    }
    // events of another device are left alive: they may still be pending
    g_events.device = dev;
    g_events.start = a;
    g_events.done = c;
  }
  *start = g_events.start;
  *done = g_events.done;
  return DSA_OK;
}

// ---- static scratch of dsa_decode_step_noalloc ------------------------------
// The workspace of the step for callers that cannot allocate: one array in
// each device's memory for the life of the process.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol); it asks the runtime for the device address once per device and
// passes that pointer to the kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

#ifdef DSA_DEVICE_CHECKS
// flags the checked kernels record (DSA_CHECK_*), one word per device
static __device__ uint32_t check_word;
#endif

namespace {

#ifdef DSA_DEVICE_CHECKS
std::mutex g_check_mu;
uint32_t* g_check_ptr[kScratchDevices] = {};
#endif

// Device address of this device's check word (NULL in normal builds, or if
// it cannot be resolved: the query call then reports the error).
uint32_t* check_word_ptr() {
#ifdef DSA_DEVICE_CHECKS
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_check_mu);
  if (!g_check_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(check_word)) != hipSuccess) return nullptr;
    g_check_ptr[dev] = static_cast<uint32_t*>(p);
  }
  return g_check_ptr[dev];
#else
  return nullptr;
#endif
}

// The batch's device view for a launch (with the check word in checked builds).
BatchArgs launch_args(const dsa_batch_t& b) {
  BatchArgs a = dsa::batch_args(b);
  a.check = check_word_ptr();
  return a;
}

// Device address of this device's scratch (resolved on the first call with
// the device current).
int scratch_on_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(DSA_ERR_UNSUPPORTED, "device ordinal beyond the static scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(DSA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

int decode_step_impl(const dsa_batch_t* batch, const dsa_indexer_inputs_t* ix,
                     const dsa_mla_inputs_t* mla, int32_t k, const dsa_step_opts_t* opts,
                     int32_t* idx_out, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                     void* stream_main, void* stream_aux);

}  // namespace

extern "C" {

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported shape";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_HIP: return "HIP error";
    case DSA_ERR_DEVICE_CHECK: return "device check failed";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return g_err.c_str(); }

int32_t dsa_device_checks_enabled(void) {
#ifdef DSA_DEVICE_CHECKS
  return 1;
#else
  return 0;
#endif
}

int dsa_device_check(uint32_t* flags_out, void* stream) {
  g_err.clear();
  if (flags_out) *flags_out = 0;
#ifdef DSA_DEVICE_CHECKS
  uint32_t* p = check_word_ptr();
  if (!p) return fail(DSA_ERR_HIP, "cannot resolve the device check word");
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  uint32_t flags = 0;
  e = hipMemcpy(&flags, p, sizeof flags, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (check word)");
  if (flags) {
    const uint32_t zero = 0;
    e = hipMemcpy(p, &zero, sizeof zero, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy (check word reset)");
    char msg[96];
    snprintf(msg, sizeof msg, "device checks found bad data (flags 0x%x)", flags);
    g_err = msg;
  }
  if (flags_out) *flags_out = flags;
  return flags ? DSA_ERR_DEVICE_CHECK : DSA_OK;
#else
  (void)stream;
  return DSA_OK;
#endif
}

int32_t dsa_default_splits(const dsa_batch_t* batch, int32_t k) {
  if (check_batch(batch) != DSA_OK || k < 1) return 1;
  return dsa::default_splits(dsa::batch_args(*batch), k);
}

int dsa_decode_layers(const dsa_batch_t* batch, int32_t n_layers, const dsa_layer_t* layers,
                      int32_t k, int32_t retention, int32_t mli, int32_t n_split, int32_t* sel,
                      void* ws, size_t ws_bytes, void* stream_main, void* stream_aux) {
  g_err.clear();
  int rc = check_batch(batch);
  if (rc) return rc;
  if (n_layers < 1 || !layers) return fail(DSA_ERR_INVALID_ARG, "need at least one layer");
  if (retention < 1) return fail(DSA_ERR_INVALID_ARG, "retention must be >= 1");
  if (mli != 0 && mli != 1) return fail(DSA_ERR_INVALID_ARG, "mli must be 0 or 1");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID_ARG, "k must be in [1, 8192]");
  if (mli && (!stream_aux || stream_aux == stream_main))
    return fail(DSA_ERR_INVALID_ARG, "MLI needs a second stream");
  int used = 1;
  rc = resolve_splits(batch, k, n_split, &used);
  if (rc) return rc;
  if (batch->num_tokens == 0) return DSA_OK;
  if (!sel) return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  const bool keys = batch->max_seqlen_k > 0;
  for (int32_t l = 0; l < n_layers; ++l) {
    const dsa_layer_t& L = layers[l];
    if (!L.out || !L.mla.q || (keys && !L.mla.kv_cache))
      return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer in a layer");
    rc = check_mla_align(L.mla.q, L.mla.kv_cache, L.out, ws);
    if (rc) return rc;
    if (l % retention == 0 && (rc = check_index_align(L.ix.q8, L.ix.k8_cache, nullptr)))
      return rc;
    if (l % retention == 0 &&
        (!L.ix.q8 || !L.ix.q_scale || !L.ix.w || (keys && (!L.ix.k8_cache || !L.ix.k_scale))))
      return fail(DSA_ERR_INVALID_ARG, "NULL indexer pointer in an indexer layer");
  }
  if (!dsa::topk_supported(dsa::batch_args(*batch), k))
    return fail(DSA_ERR_UNSUPPORTED, "rows longer than 393216 tokens need k <= 4096");
  const StepWs W = step_layout(batch, used);
  if (ws_bytes < W.total || !ws) return fail(DSA_ERR_WORKSPACE, "step workspace too small");

  const dsa::BatchArgs a = launch_args(*batch);
  const int64_t per = (int64_t)batch->num_tokens * k;
  void* mla_ws = static_cast<char*>(ws) + W.mla_off;
  for (int32_t l = 0; l < n_layers; ++l) {
    const dsa_layer_t& L = layers[l];
    const int64_t j = l / retention;
    int32_t* latest = sel + j * per;
    if (l % retention == 0) {
      dsa_step_opts_t o{};
      o.n_split = n_split;
      if (mli && l > 0) {
        o.mode = DSA_MODE_MLI;
        o.attend_idx = sel + (j - 1) * per;
      } else {
        o.mode = DSA_MODE_FUSED;
      }
      rc = dsa_decode_step(batch, &L.ix, &L.mla, k, &o, latest, L.out, L.lse, ws, ws_bytes,
                           stream_main, stream_aux);
      if (rc) return rc;
    } else {
      // a layer without an indexer attends the latest indexer layer's selection
      hipError_t e = dsa::launch_sparse_mla(a, L.mla.q, L.mla.kv_cache, latest, k,
                                            L.mla.sm_scale, L.out, L.lse, used, mla_ws,
                                            (hipStream_t)stream_main);
      if (e != hipSuccess) return hip_fail(e, "sparse MLA launch");
    }
  }
  return DSA_OK;
}

size_t dsa_workspace_size(int op, const dsa_batch_t* batch, int32_t k, int32_t n_split) {
  if (check_batch(batch) != DSA_OK || k < 1 || k > DSA_MAX_TOPK) return 0;
  const BatchArgs a = dsa::batch_args(*batch);
  int used = 1;
  switch (op) {
    case DSA_OP_TOPK:
      return dsa::topk_ws_layout(a).total;
    case DSA_OP_SPARSE_MLA:
      if (resolve_splits(batch, k, n_split, &used) != DSA_OK) return 0;
      return dsa::mla_ws_layout(a, used).total;
    case DSA_OP_DECODE_STEP:
      if (resolve_splits(batch, k, n_split, &used) != DSA_OK) return 0;
      return step_layout(batch, used).total;
    case DSA_OP_MASKED_MHA:
      return dsa::mha_supported(a) ? dsa::mha_ws_layout(a).total : 0;
    case DSA_OP_DENSE_MLA:
      if (resolve_splits(batch, std::max(1, batch->max_seqlen_k), n_split, &used) != DSA_OK ||
          used > dsa::kMaxSplits)
        return 0;
      return dsa::mla_ws_layout(a, used).total;
    default:
      return 0;
  }
}

int dsa_index_score(const dsa_batch_t* batch, const uint8_t* q8, const float* q_scale,
                    const float* w, const uint8_t* k8_cache, const float* k_scale, float* scores,
                    int64_t ld, void* stream) {
  g_err.clear();
  int rc = check_batch(batch);
  if (rc) return rc;
  if (ld < batch->max_seqlen_k) return fail(DSA_ERR_INVALID_ARG, "ld < max_seqlen_k");
  if (batch->num_tokens == 0 || batch->max_seqlen_k == 0) return DSA_OK;
  if (!q8 || !q_scale || !w || !k8_cache || !k_scale || !scores)
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  rc = check_index_align(q8, k8_cache, scores);
  if (rc) return rc;
  hipError_t e = dsa::launch_index_score(launch_args(*batch), q8, q_scale, w, k8_cache,
                                         k_scale, scores, ld, nullptr, (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "index_score launch");
}

int dsa_cache_append(const dsa_batch_t* batch, const uint16_t* k_new, const uint16_t* kv_new,
                     uint8_t* k8_cache, float* k_scale, uint16_t* kv_cache, void* stream) {
  g_err.clear();
  int rc = check_batch(batch);
  if (rc) return rc;
  if (batch->num_tokens == 0 || batch->max_seqlen_k == 0) return DSA_OK;
  if (!k_new || !kv_new || !k8_cache || !k_scale || !kv_cache)
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  auto misaligned = [](const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) != 0; };
  if (misaligned(kv_new, 16) || misaligned(kv_cache, 16) || misaligned(k_new, 4) ||
      misaligned(k8_cache, 2) || misaligned(k_scale, 4))
    return fail(DSA_ERR_INVALID_ARG,
                "kv_new / kv_cache need 16-byte, k_new / k_scale 4-byte, k8_cache 2-byte alignment");
  hipError_t e = dsa::launch_cache_append(launch_args(*batch), k_new, kv_new, k8_cache, k_scale,
                                          kv_cache, (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "cache_append launch");
}

namespace {

int topk_common(const dsa_batch_t* batch, const float* scores, int64_t ld, int32_t k, int32_t space,
                const int32_t* kv_offsets, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  int rc = check_batch(batch);
  if (rc) return rc;
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID_ARG, "k must be in [1, 8192]");
  if (ld < batch->max_seqlen_k) return fail(DSA_ERR_INVALID_ARG, "ld < max_seqlen_k");
  if (space != DSA_IDX_LOGICAL && space != DSA_IDX_PAGED && space != DSA_IDX_RAGGED)
    return fail(DSA_ERR_INVALID_ARG, "unknown index space");
  if (batch->num_tokens == 0) return DSA_OK;
  if (!idx || (!scores && batch->max_seqlen_k > 0))
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (space == DSA_IDX_RAGGED && !kv_offsets)
    return fail(DSA_ERR_INVALID_ARG, "ragged indices need kv_offsets");
  if (!dsa::topk_supported(dsa::batch_args(*batch), k))
    return fail(DSA_ERR_UNSUPPORTED, "rows longer than 393216 tokens need k <= 4096");
  const size_t need = dsa::topk_ws_layout(dsa::batch_args(*batch)).total;
  if (ws_bytes < need || !ws) return fail(DSA_ERR_WORKSPACE, "top-k workspace too small");
  if (misaligned16(ws)) return fail(DSA_ERR_INVALID_ARG, "ws needs 16-byte alignment");
  hipError_t e = dsa::launch_topk(launch_args(*batch), scores, ld, k, idx, ws,
                                  (hipStream_t)stream, space, kv_offsets);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "top-k launch");
}

int mla_common(const dsa_batch_t* batch, const uint16_t* q, const uint16_t* kv_cache,
               const int32_t* idx, int32_t k, float sm_scale, uint16_t* out, float* lse,
               int32_t n_split, void* ws, size_t ws_bytes, void* stream, int idx_mode) {
  g_err.clear();
  int rc = check_batch(batch);
  if (rc) return rc;
  if (idx_mode == dsa::kMlaDense) {
    k = std::max(1, batch->max_seqlen_k);  // the dense form attends every visible position
  } else if (k < 1 || k > DSA_MAX_TOPK) {
    return fail(DSA_ERR_INVALID_ARG, "k must be in [1, 8192]");
  }
  int used = 1;
  rc = resolve_splits(batch, k, n_split, &used);
  if (rc) return rc;
  if (used > dsa::kMaxSplits)
    return fail(DSA_ERR_UNSUPPORTED, "dense attention covers at most 131072 tokens per row");
  if (batch->num_tokens == 0) return DSA_OK;
  if (!q || !out || (!idx && idx_mode != dsa::kMlaDense) ||
      (!kv_cache && (batch->max_seqlen_k > 0 || idx_mode == dsa::kMlaPaged)))
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  rc = check_mla_align(q, kv_cache, out, ws);
  if (rc) return rc;
  const dsa::BatchArgs a = launch_args(*batch);
  const size_t need = dsa::mla_ws_layout(a, used).total;
  if (need > 0 && (ws_bytes < need || !ws))
    return fail(DSA_ERR_WORKSPACE, "attention workspace too small");
  hipError_t e = dsa::launch_sparse_mla(a, q, kv_cache, idx, k, sm_scale, out, lse, used, ws,
                                        (hipStream_t)stream, idx_mode);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "sparse MLA launch");
}

}  // namespace

int dsa_topk(const dsa_batch_t* batch, const float* scores, int64_t ld, int32_t k, int32_t* idx,
             void* ws, size_t ws_bytes, void* stream) {
  return topk_common(batch, scores, ld, k, DSA_IDX_LOGICAL, nullptr, idx, ws, ws_bytes, stream);
}

int dsa_topk_transform(const dsa_batch_t* batch, const float* scores, int64_t ld, int32_t k,
                       int32_t space, const int32_t* kv_offsets, int32_t* idx, void* ws,
                       size_t ws_bytes, void* stream) {
  return topk_common(batch, scores, ld, k, space, kv_offsets, idx, ws, ws_bytes, stream);
}

int dsa_sparse_mla_decode(const dsa_batch_t* batch, const uint16_t* q, const uint16_t* kv_cache,
                          const int32_t* idx, int32_t k, float sm_scale, uint16_t* out,
                          float* lse, int32_t n_split, void* ws, size_t ws_bytes, void* stream) {
  return mla_common(batch, q, kv_cache, idx, k, sm_scale, out, lse, n_split, ws, ws_bytes, stream,
                    dsa::kMlaLogical);
}

int dsa_dense_mla_decode(const dsa_batch_t* batch, const uint16_t* q, const uint16_t* kv_cache,
                         float sm_scale, uint16_t* out, float* lse, int32_t n_split, void* ws,
                         size_t ws_bytes, void* stream) {
  return mla_common(batch, q, kv_cache, nullptr, 0, sm_scale, out, lse, n_split, ws, ws_bytes,
                    stream, dsa::kMlaDense);
}

int dsa_masked_mha_prefill(const dsa_batch_t* batch, const uint16_t* q_nope,
                           const uint16_t* q_rope, const uint16_t* w_uk, const uint16_t* w_uv,
                           const uint16_t* kv_cache, const int32_t* idx, int32_t k,
                           float sm_scale, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                           void* stream) {
  g_err.clear();
  int rc = check_batch(batch);
  if (rc) return rc;
  if (idx && (k < 1 || k > DSA_MAX_TOPK)) return fail(DSA_ERR_INVALID_ARG, "k must be in [1, 8192]");
  const dsa::BatchArgs a = launch_args(*batch);
  if (!dsa::mha_supported(a))
    return fail(DSA_ERR_UNSUPPORTED, "the masked MHA form covers at most 65536 tokens per row");
  if (batch->num_tokens == 0) return DSA_OK;
  if (!q_nope || !q_rope || !w_uk || !w_uv || !out ||
      (!kv_cache && batch->max_seqlen_k > 0))
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  if (misaligned16(q_nope) || misaligned16(q_rope) || misaligned16(w_uk) || misaligned16(w_uv) ||
      misaligned16(kv_cache) || misaligned16(out) || misaligned16(ws))
    return fail(DSA_ERR_INVALID_ARG, "q_nope, q_rope, w_uk, w_uv, kv_cache, out and ws need "
                                     "16-byte alignment");
  const size_t need = dsa::mha_ws_layout(a).total;
  if (ws_bytes < need || !ws) return fail(DSA_ERR_WORKSPACE, "masked MHA workspace too small");
  hipError_t e = dsa::launch_masked_mha(a, q_nope, q_rope, w_uk, w_uv, kv_cache, idx, idx ? k : 0,
                                        sm_scale, out, lse, ws, (hipStream_t)stream);
  return e == hipSuccess ? DSA_OK : hip_fail(e, "masked MHA launch");
}

int dsa_sparse_mla_decode_paged(const dsa_batch_t* batch, const uint16_t* q,
                                const uint16_t* kv_cache, const int32_t* slots, int32_t k,
                                float sm_scale, uint16_t* out, float* lse, int32_t n_split,
                                void* ws, size_t ws_bytes, void* stream) {
  return mla_common(batch, q, kv_cache, slots, k, sm_scale, out, lse, n_split, ws, ws_bytes, stream,
                    dsa::kMlaPaged);
}

int dsa_decode_step(const dsa_batch_t* batch, const dsa_indexer_inputs_t* ix,
                    const dsa_mla_inputs_t* mla, int32_t k, const dsa_step_opts_t* opts,
                    int32_t* idx_out, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                    void* stream_main, void* stream_aux) {
  g_err.clear();
  return decode_step_impl(batch, ix, mla, k, opts, idx_out, out, lse, ws, ws_bytes, stream_main,
                          stream_aux);
}

int dsa_decode_step_noalloc(const dsa_batch_t* batch, const dsa_indexer_inputs_t* ix,
                            const dsa_mla_inputs_t* mla, int32_t k, const dsa_step_opts_t* opts,
                            int32_t* idx_out, uint16_t* out, float* lse, void* stream) {
  g_err.clear();
  int rc = check_batch(batch);
  if (rc) return rc;
  if (!opts) return fail(DSA_ERR_INVALID_ARG, "NULL argument struct");
  if (opts->mode != DSA_MODE_FUSED)
    return fail(DSA_ERR_INVALID_ARG, "dsa_decode_step_noalloc runs FUSED steps only");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID_ARG, "k must be in [1, 8192]");
  int used = 1;
  rc = resolve_splits(batch, k, opts->n_split, &used);
  if (rc) return rc;
  if (batch->num_tokens == 0) return DSA_OK;
  const size_t need = step_layout(batch, used).total;
  if (need > kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof msg,
             "the step needs %zu bytes of workspace; the static scratch holds 64 MiB "
             "(use dsa_decode_step with a caller workspace)", need);
    return fail(DSA_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  rc = scratch_on_device(&ws);
  if (rc) return rc;
  return decode_step_impl(batch, ix, mla, k, opts, idx_out, out, lse, ws, kScratchBytes, stream,
                          nullptr);
}

}  // extern "C"

namespace {

int decode_step_impl(const dsa_batch_t* batch, const dsa_indexer_inputs_t* ix,
                     const dsa_mla_inputs_t* mla, int32_t k, const dsa_step_opts_t* opts,
                     int32_t* idx_out, uint16_t* out, float* lse, void* ws, size_t ws_bytes,
                     void* stream_main, void* stream_aux) {
  int rc = check_batch(batch);
  if (rc) return rc;
  if (!ix || !mla || !opts) return fail(DSA_ERR_INVALID_ARG, "NULL argument struct");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID_ARG, "k must be in [1, 8192]");
  if (opts->mode != DSA_MODE_FUSED && opts->mode != DSA_MODE_MLI)
    return fail(DSA_ERR_INVALID_ARG, "unknown mode");
  const bool mli = opts->mode == DSA_MODE_MLI;
  if (mli && (!opts->attend_idx || !stream_aux || stream_aux == stream_main))
    return fail(DSA_ERR_INVALID_ARG, "MLI mode needs attend_idx and a second stream");
  if (mli && idx_out) {
    // the aux stream writes idx_out while the main stream reads attend_idx
    const uintptr_t a0 = (uintptr_t)opts->attend_idx, i0 = (uintptr_t)idx_out;
    const uintptr_t n = (uintptr_t)batch->num_tokens * (uintptr_t)k * sizeof(int32_t);
    if (n > 0 && a0 < i0 + n && i0 < a0 + n)
      return fail(DSA_ERR_INVALID_ARG, "attend_idx overlaps idx_out in MLI mode");
  }
  // in MLI mode the attention shares the GPU with the scan on the other
  // stream: by default it takes half the CUs (the ragged 96-row batch: two
  // streams 0.226 ms with 1 split, 0.243 ms with 2)
  int used = 1;
  rc = resolve_splits(batch, k, opts->n_split, &used, mli ? dsa::kAttnWGsShared : dsa::kAttnWGs);
  if (rc) return rc;
  if (batch->num_tokens == 0) return DSA_OK;
  if (!idx_out || !out || !mla->q || !ix->q8 || !ix->q_scale || !ix->w ||
      (batch->max_seqlen_k > 0 && (!ix->k8_cache || !ix->k_scale || !mla->kv_cache)))
    return fail(DSA_ERR_INVALID_ARG, "NULL tensor pointer");
  rc = check_mla_align(mla->q, mla->kv_cache, out, ws);
  if (rc) return rc;
  rc = check_index_align(ix->q8, ix->k8_cache, nullptr);
  if (rc) return rc;
  if (!dsa::topk_supported(dsa::batch_args(*batch), k))
    return fail(DSA_ERR_UNSUPPORTED, "rows longer than 393216 tokens need k <= 4096");
  const StepWs L = step_layout(batch, used);
  if (ws_bytes < L.total || !ws) return fail(DSA_ERR_WORKSPACE, "step workspace too small");
  const BatchArgs a = launch_args(*batch);
  char* base = static_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(base + L.scores_off);
  void* topk_ws = base + L.topk_off;
  void* mla_ws = base + L.mla_off;
  const int64_t ld = step_ld(batch);
  hipStream_t sm = (hipStream_t)stream_main;

  // indexer + top-k on stream s: the scan also builds the first radix
  // histogram of each row, so the top-k starts at its threshold step
  // optional stage events: mark(i, 0) before stage i, mark(i, 1) after it
  auto mark = [&](int stage, int end, hipStream_t s) -> hipError_t {
    if (!opts->stage_events) return hipSuccess;
    return hipEventRecord((hipEvent_t)opts->stage_events[2 * stage + end], s);
  };

  // rows whose visible tokens all fit in k select every one of them: no
  // scan is needed (the short-context dense form); the attention then takes
  // the positions in order, exactly as it would from the top-k's output
  const bool dense = batch->max_seqlen_k <= k;
  auto select = [&](hipStream_t s) -> int {
    hipError_t e;
    if (dense) {
      if ((e = mark(DSA_STAGE_INDEX_SCORE, 0, s)) != hipSuccess ||
          (e = mark(DSA_STAGE_INDEX_SCORE, 1, s)) != hipSuccess ||
          (e = mark(DSA_STAGE_TOPK, 0, s)) != hipSuccess)
        return hip_fail(e, "hipEventRecord");
      e = dsa::launch_select_all(a, k, idx_out, s);
      if (e != hipSuccess) return hip_fail(e, "select launch");
      if ((e = mark(DSA_STAGE_TOPK, 1, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      return DSA_OK;
    }
    // rows short enough for the one-pass top-k need no histogram from the
    // scan (nor the zeroed workspace it accumulates into)
    const bool rows = dsa::topk_rows_fit(a, scores, ld);
    if (!rows) {
      e = dsa::launch_topk_zero(a, topk_ws, s);
      if (e != hipSuccess) return hip_fail(e, "top-k zero launch");
    }
    if ((e = mark(DSA_STAGE_INDEX_SCORE, 0, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    e = dsa::launch_index_score(a, ix->q8, ix->q_scale, ix->w, ix->k8_cache, ix->k_scale, scores,
                                ld, rows ? nullptr : dsa::topk_hist1(a, topk_ws), s, mli);
    if (e != hipSuccess) return hip_fail(e, "index_score launch");
    if ((e = mark(DSA_STAGE_INDEX_SCORE, 1, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = mark(DSA_STAGE_TOPK, 0, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    e = rows ? dsa::launch_topk_rows(a, scores, ld, k, idx_out, s)
             : dsa::launch_topk_select(a, scores, ld, k, idx_out, topk_ws, s);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
    if ((e = mark(DSA_STAGE_TOPK, 1, s)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    return DSA_OK;
  };
  auto attend = [&](const int32_t* sel, int idx_mode) -> int {
    hipError_t e = mark(DSA_STAGE_ATTENTION, 0, sm);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    e = dsa::launch_sparse_mla(a, mla->q, mla->kv_cache, sel, k, mla->sm_scale, out, lse, used,
                               mla_ws, sm, idx_mode);
    if (e != hipSuccess) return hip_fail(e, "sparse MLA launch");
    if ((e = mark(DSA_STAGE_ATTENTION, 1, sm)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    return DSA_OK;
  };

  if (!mli) {
    rc = select(sm);
    if (rc) return rc;
    // the selection just written is compact (positions first, then -1)
    return attend(idx_out, dense ? dsa::kMlaDense : dsa::kMlaCompact);
  }

  // MLI: attention over the previous indexer layer's selection on the main
  // stream, this layer's indexer + top-k on the aux stream, joined at the end
  hipStream_t sa = (hipStream_t)stream_aux;
  hipEvent_t ev_start, ev_done;
  rc = get_events(&ev_start, &ev_done);
  if (rc) return rc;
  hipError_t e = hipEventRecord(ev_start, sm);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  e = hipStreamWaitEvent(sa, ev_start, 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  rc = select(sa);
  if (rc) return rc;
  rc = attend(opts->attend_idx, dsa::kMlaLogical);
  if (rc) return rc;
  e = hipEventRecord(ev_done, sa);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  e = hipStreamWaitEvent(sm, ev_done, 0);
  if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  return DSA_OK;
}

}  // namespace
