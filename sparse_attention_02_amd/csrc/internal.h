// Internal launch interface between the C-ABI layer (api.cpp) and the HIP
// kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "dsa.h"

namespace dsa {

// Device view of the batch metadata; host scalars copied by value.
struct BatchArgs {
  int32_t B, T, max_q, max_seqlen_k, max_pages, num_pages;
  const int32_t* cu;     // [B+1]
  const int32_t* lens;   // [B]
  const int32_t* pages;  // [B, max_pages]
  uint32_t* check;       // device check word (builds with DSA_DEVICE_CHECKS), else NULL
};

inline BatchArgs batch_args(const dsa_batch_t& b) {
  return BatchArgs{b.batch,        b.num_tokens,   b.max_q,     b.max_seqlen_k,
                   b.max_pages_per_req, b.num_pages, b.cu_seqlens_q, b.seqlens_k,
                   b.page_table, nullptr};
}

constexpr int kTopkBins = 2048;      // first radix digit: key bits 31..21
constexpr int kTopkSeg = 8192;       // scores per work-group of the standalone histogram pass
constexpr int kMlaTile = 32;         // selected tokens per attention tile
constexpr int kMaxSplits = 64;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace carve-up of the top-k (all sizes in bytes).
struct TopkWs {
  size_t hist_off, ctrl_off, cand_off, total;
};
TopkWs topk_ws_layout(const BatchArgs& b);

struct MlaWs {
  size_t opart_off, spart_off, lpart_off, total;
};
MlaWs mla_ws_layout(const BatchArgs& b, int n_split);

// KV splits for n_split = 0: at most `wgs` work-groups of the attention
// (256 fill the CUs; beside a concurrent scan, fewer leave it room).
constexpr int kAttnWGs = 256;
constexpr int kAttnWGsShared = 128;
int default_splits(const BatchArgs& b, int k, int wgs = kAttnWGs);

// KV splits actually launched for k tokens per row and a requested split count.
int mla_splits_used(int k, int n_split);

// hist (may be NULL): per-row histogram of the top 11 bits of each score's
// order-preserving key, [T][kTopkBins], accumulated with atomics.
// shared: the scan runs beside another kernel (multi-layer-indexer mode) and
// uses smaller work-groups.
hipError_t launch_index_score(const BatchArgs& b, const uint8_t* q8, const float* q_scale,
                              const float* w, const uint8_t* k8, const float* k_scale,
                              float* scores, int64_t ld, uint32_t* hist, hipStream_t s,
                              bool shared = false);

// Whole top-k: zero, histogram, threshold, collect, final.
// space: DSA_IDX_LOGICAL / PAGED / RAGGED (kv_off [B] for RAGGED, else unused)
hipError_t launch_topk(const BatchArgs& b, const float* scores, int64_t ld, int k, int32_t* idx,
                       void* ws, hipStream_t s, int space = DSA_IDX_LOGICAL,
                       const int32_t* kv_off = nullptr);
// Pieces used by the fused step, whose indexer builds the histogram.
hipError_t launch_topk_zero(const BatchArgs& b, void* ws, hipStream_t s);
hipError_t launch_topk_select(const BatchArgs& b, const float* scores, int64_t ld, int k,
                              int32_t* idx, void* ws, hipStream_t s, int space = DSA_IDX_LOGICAL,
                              const int32_t* kv_off = nullptr);
uint32_t* topk_hist1(const BatchArgs& b, void* ws);
// Rows of at most 65536 positions with 16-byte aligned rows: one launch,
// one work-group per row, no workspace and no histogram from the scan.
bool topk_rows_fit(const BatchArgs& b, const float* scores, int64_t ld);
hipError_t launch_topk_rows(const BatchArgs& b, const float* scores, int64_t ld, int k,
                            int32_t* idx, hipStream_t s, int space = DSA_IDX_LOGICAL,
                            const int32_t* kv_off = nullptr);
bool topk_supported(const BatchArgs& b, int k);

hipError_t launch_cache_append(const BatchArgs& b, const uint16_t* k_new, const uint16_t* kv_new,
                               uint8_t* k8, float* ks, uint16_t* kv, hipStream_t s);

// What the attention's idx holds: logical positions, physical slots, or
// nothing (dense: every visible position among the first k, idx unused).
// kMlaCompact: logical positions whose row holds its min(k, v) entries first
// and -1 after (the top-k's own output), so later entries are not read.
enum MlaIndex { kMlaLogical = 0, kMlaPaged = 1, kMlaDense = 2, kMlaCompact = 3 };
hipError_t launch_sparse_mla(const BatchArgs& b, const uint16_t* q, const uint16_t* kv,
                             const int32_t* idx, int k, float sm_scale, uint16_t* out, float* lse,
                             int n_split, void* ws, hipStream_t s, int idx_mode = kMlaLogical);

// idx[t, j] = j for j < v_t (j < k), -1 after: the selection of a row whose
// visible tokens all fit in k.
// Masked multi-head attention (expanded form): workspace of the expanded
// keys and values [B][H][lp][128], the rope dims [B][lp][64] (bf16) and the
// attend mask [T][lp/32] (lp: max_seqlen_k rounded up to 64).
struct MhaWs {
  size_t kn_off, vn_off, rope_off, mask_off, total;
  int lp, nwords;
};
MhaWs mha_ws_layout(const BatchArgs& b);
bool mha_supported(const BatchArgs& b);  // rows of at most 65536 positions
hipError_t launch_masked_mha(const BatchArgs& b, const uint16_t* q_nope, const uint16_t* q_rope,
                             const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* kv,
                             const int32_t* idx, int k, float sm_scale, uint16_t* out,
                             float* lse, void* ws, hipStream_t s);

hipError_t launch_select_all(const BatchArgs& b, int k, int32_t* idx, hipStream_t s);

}  // namespace dsa
