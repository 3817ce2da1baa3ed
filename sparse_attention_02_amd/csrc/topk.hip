// Per-row top-k for gfx950: radix select on order-preserving uint32 keys.
//
// Each row keeps the K = min(k, v_t) visible positions with the largest
// scores; at the k-th score ties go to the lower position ("MTP and sparse
// attention: NSA and DSA", DSA bullet: each query keeps its top 2048).
//
//   1. hist1   per-row histogram of the top 11 key bits (LDS histograms added
//              into global memory).  The fused decode step builds it inside
//              the indexer scan instead (no extra pass over the scores).
//   2. collect (row x 8192-score segment): each work-group finds the bin b1
//              holding the K-th largest key from hist1 (while its score loads
//              are in flight); keys in bins above b1 are selected outright,
//              keys in b1 become candidates; one atomic per work-group
//              reserves the output ranges, ranks inside the work-group come
//              from a block scan.  It also histograms bits 20..10 of the
//              candidates (hist2).
//   3. final   (row): the second digit from hist2, the third from one pass
//              over the candidates, ties at the exact threshold resolved by
//              a radix select on the position (lowest positions win), then
//              the K positions are written in ascending order (LDS bitmap,
//              or a bitonic sort for rows longer than the bitmap).
// The output is deterministic: the selected set in ascending order.
#include "device_common.h"

namespace dsa {
namespace {

constexpr int kHistThreads = 256;
constexpr int kCollectThreads = 256;
constexpr int kPerThread = kTopkSeg / kCollectThreads;  // 32 scores per thread
constexpr int kFinalThreads = 1024;
constexpr int kBitmapWords = 12288;  // 48 KB: rows up to 393216 positions
constexpr int kSortCap = 4096;       // bitonic fallback (rows longer than the bitmap)

// ctrl words per row
constexpr int kCtrlB1 = 0;     // threshold bin (-1: every visible position selected)
constexpr int kCtrlAbove = 1;  // positions written as "above"
constexpr int kCtrlCand = 2;   // candidates appended
constexpr int kCtrlWords = 4;

__global__ void zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__device__ __forceinline__ int row_len(const BatchArgs& b, int t) {
  const int bi = row_request(b.cu, b.B, t);
  return row_visible(b, bi, t);
}

__global__ __launch_bounds__(kHistThreads) void topk_hist_kernel(BatchArgs b,
                                                                  const float* __restrict__ scores,
                                                                  int64_t ld, int k,
                                                                  uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[kTopkBins];
  const int t = blockIdx.x;
  const int v = row_len(b, t);
  if (v <= k) return;  // every position is selected; no histogram needed
  const int s0 = blockIdx.y * kTopkSeg;
  if (s0 >= v) return;
  const int s1 = min(v, s0 + kTopkSeg);
  for (int i = threadIdx.x; i < kTopkBins; i += kHistThreads) h[i] = 0u;
  __syncthreads();
  const float* row = scores + (int64_t)t * ld;
  // batches of 8 independent loads per thread
  for (int base = s0; base < s1; base += 8 * kHistThreads) {
    uint32_t kk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      kk[u] = float_key(row[min(base + (int)threadIdx.x + u * kHistThreads, s1 - 1)]);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (base + (int)threadIdx.x + u * kHistThreads < s1) atomicAdd(&h[kk[u] >> 21], 1u);
  }
  __syncthreads();
  uint32_t* gh = hist + (int64_t)t * kTopkBins;
  for (int i = threadIdx.x; i < kTopkBins; i += kHistThreads)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Largest bin `bin` of h[0..nbins) with sum_{b > bin} h[b] < need <=
// sum_{b >= bin} h[b]; *above = sum_{b > bin} h[b].  Block-wide; need >= 1
// and sum h >= need.  `scan` is LDS scratch of blockDim.x words.
__device__ void find_cut(const uint32_t* h, int nbins, uint32_t need, int* bin, uint32_t* above,
                         uint32_t* scan) {
  const int nt = blockDim.x;
  const int per = (nbins + nt - 1) / nt;
  const int lo = threadIdx.x * per;
  const int hi = min(nbins, lo + per);
  uint32_t mine = 0;
  for (int i = lo; i < hi; ++i) mine += h[i];
  scan[threadIdx.x] = mine;
  __syncthreads();
  // inclusive suffix sum over threads (Hillis-Steele)
  for (int off = 1; off < nt; off <<= 1) {
    uint32_t add = threadIdx.x + off < nt ? scan[threadIdx.x + off] : 0u;
    __syncthreads();
    scan[threadIdx.x] += add;
    __syncthreads();
  }
  uint32_t run = scan[threadIdx.x] - mine;  // sum of bins above this thread's range
  for (int i = hi - 1; i >= lo; --i) {
    const uint32_t c = h[i];
    if (run < need && run + c >= need) {
      *bin = i;
      *above = run;
    }
    run += c;
  }
  __syncthreads();
}

// Exclusive prefix sum of x over the block (blockDim.x a multiple of 64,
// at most 1024 threads); *total receives the sum.  `wsum` holds 16 words.
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t x, uint32_t* wsum,
                                                        uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
  for (int w = 0; w < nw; ++w) {
    const uint32_t s = wsum[w];
    if (w < wave) before += s;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + inc - x;
}

__global__ __launch_bounds__(kCollectThreads) void topk_collect_kernel(
    BatchArgs b, const float* __restrict__ scores, int64_t ld, int k,
    const uint32_t* __restrict__ hist1, int32_t* __restrict__ ctrl, int32_t* __restrict__ idx,
    uint2* __restrict__ cand, int64_t cand_stride, uint32_t* __restrict__ hist2) {
  __shared__ uint32_t h1[kTopkBins];
  __shared__ uint32_t h2[kTopkBins];
  __shared__ uint32_t scan[kCollectThreads];
  __shared__ uint32_t wsum[16];
  __shared__ uint32_t s_base[2];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  const int t = blockIdx.x;
  const int v = row_len(b, t);
  const int s0 = blockIdx.y * kTopkSeg;
  if (s0 >= v) return;
  const float* row = scores + (int64_t)t * ld;
  const bool all = v <= k;  // every visible position is selected

  // the row's first-digit histogram, then the segment's scores: element j
  // of this thread is position s0 + tid + 256 j (coalesced loads, all
  // issued before any is used: positions past the row re-read its last
  // score and are masked below).  The threshold search below runs while
  // the score loads are in flight.
  constexpr int kHistPer = kTopkBins / kCollectThreads;
  uint32_t hv[kHistPer];
#pragma unroll
  for (int i = 0; i < kHistPer; ++i)
    hv[i] = all ? 0u : hist1[(int64_t)t * kTopkBins + threadIdx.x + i * kCollectThreads];
  uint32_t key[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    key[j] = float_key(row[min(s0 + (int)threadIdx.x + j * kCollectThreads, v - 1)]);
#pragma unroll
  for (int i = 0; i < kHistPer; ++i) {
    h1[threadIdx.x + i * kCollectThreads] = hv[i];
    h2[threadIdx.x + i * kCollectThreads] = 0u;
  }
  __syncthreads();
  // b1: the first-digit bin holding the K-th largest key (-1: all selected);
  // every segment of the row finds the same bin, the first records it
  int b1 = -1;
  if (!all) {
    // (a histogram holding fewer than k keys -- scores never written for a
    // page with an invalid id -- leaves the bin at -1; the writes below stay
    // inside the row's k slots either way)
    if (threadIdx.x == 0) s_bin = -1;
    find_cut(h1, kTopkBins, (uint32_t)k, &s_bin, &s_above, scan);
    b1 = s_bin;
  }
  if (blockIdx.y == 0 && threadIdx.x == 0) ctrl[t * kCtrlWords + kCtrlB1] = b1;
  uint32_t am = 0, em = 0;  // bit j: element j is above / a candidate
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int s = s0 + threadIdx.x + j * kCollectThreads;
    const int d = (int)(key[j] >> 21);
    if (s < v) {
      if (b1 < 0 || d > b1) am |= 1u << j;
      else if (d == b1) em |= 1u << j;
    }
  }
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (em & (1u << j)) atomicAdd(&h2[(key[j] >> 10) & (kTopkBins - 1)], 1u);

  uint32_t tot_a, tot_e;
  const uint32_t ex_a = block_exclusive_sum(__popc(am), wsum, &tot_a);
  const uint32_t ex_e = block_exclusive_sum(__popc(em), wsum, &tot_e);
  if (threadIdx.x == 0) {
    s_base[0] = tot_a ? atomicAdd(&ctrl[t * kCtrlWords + kCtrlAbove], (int)tot_a) : 0;
    s_base[1] = tot_e ? atomicAdd(&ctrl[t * kCtrlWords + kCtrlCand], (int)tot_e) : 0;
  }
  __syncthreads();
  int32_t* out = idx + (int64_t)t * k;
  const uint32_t ra = s_base[0] + ex_a;  // rank of this thread's first "above" position
  uint2* cl = cand + (int64_t)t * cand_stride + s_base[1] + ex_e;
  int na = 0, ne = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int s = s0 + threadIdx.x + j * kCollectThreads;
    if (am & (1u << j)) {
      if (ra + na < (uint32_t)k) out[ra + na] = s;
      ++na;
    }
    if (em & (1u << j)) cl[ne++] = make_uint2(key[j], (uint32_t)s);
  }
  if (b1 >= 0) {
    uint32_t* gh = hist2 + (int64_t)t * kTopkBins;
    for (int i = threadIdx.x; i < kTopkBins; i += kCollectThreads)
      if (h2[i]) atomicAdd(&gh[i], h2[i]);
  }
}

// Calls f(c) for every candidate c in cl[0..n), with each thread's loads
// issued in batches of 8 before any is used.
template <typename F>
__device__ __forceinline__ void for_each_cand(const uint2* __restrict__ cl, int n, F f) {
  for (int base = 0; base < n; base += 8 * (int)blockDim.x) {
    uint2 c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = cl[min(base + (int)threadIdx.x + u * (int)blockDim.x, n - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (base + (int)threadIdx.x + u * (int)blockDim.x < n) f(c[u]);
  }
}

// Threshold x* of the `need` largest values among the items accepted by
// `get` (3 radix passes of 11, 11, 10 bits): count(x > x*) < need <=
// count(x >= x*).  Returns x*; *gt receives count(x > x*).
template <typename Get>
__device__ uint32_t radix_select(int n, uint32_t need, Get get, uint32_t* h, uint32_t* scan,
                                 int* s_bin, uint32_t* s_above, uint32_t* gt) {
  uint32_t prefix = 0;
  uint32_t done_above = 0;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const int nb = 1 << widths[pass];
    const int hs = sh + widths[pass];  // bits above this digit must match prefix
    for (int i = threadIdx.x; i < nb; i += blockDim.x) h[i] = 0u;
    __syncthreads();
    for (int base = 0; base < n; base += 4 * (int)blockDim.x) {
      uint32_t xs[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) ok[u] = get(min(base + (int)threadIdx.x + u * (int)blockDim.x, n - 1), &xs[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (base + (int)threadIdx.x + u * (int)blockDim.x >= n || !ok[u]) continue;
        if (hs < 32 && (xs[u] >> hs) != (prefix >> hs)) continue;
        atomicAdd(&h[(xs[u] >> sh) & (nb - 1)], 1u);
      }
    }
    __syncthreads();
    find_cut(h, nb, need - done_above, s_bin, s_above, scan);
    prefix |= (uint32_t)(*s_bin) << sh;
    done_above += *s_above;
    __syncthreads();
  }
  *gt = done_above;
  return prefix;
}

// The index a selected position is reported as: itself (DSA_IDX_LOGICAL),
// its physical slot through the page table (DSA_IDX_PAGED; -1 for a page id
// outside the pool), or its offset in a ragged buffer that holds request b's
// tokens from kv_off[b] on (DSA_IDX_RAGGED).
__device__ __forceinline__ int32_t index_in_space(const BatchArgs& b, int bi, int space,
                                                  const int32_t* kv_off, int pos) {
  if (space == DSA_IDX_PAGED) return (int32_t)slot_of(b, bi, pos);
  if (space == DSA_IDX_RAGGED) return kv_off[bi] + pos;
  return pos;
}

__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(
    BatchArgs b, int k, const int32_t* __restrict__ ctrl, const uint32_t* __restrict__ hist2,
    int32_t* __restrict__ idx, const uint2* __restrict__ cand, int64_t cand_stride, int space,
    const int32_t* __restrict__ kv_off) {
  __shared__ uint32_t bitmap[kBitmapWords];
  __shared__ int32_t sel[kSortCap];
  __shared__ uint32_t h[kTopkBins];
  __shared__ uint32_t scan[kFinalThreads];
  __shared__ uint32_t wsum[16];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  __shared__ int32_t s_count;
  const int t = blockIdx.x;
  const int bi = row_request(b.cu, b.B, t);
  const int v = row_visible(b, bi, t);
  const int K = min(k, v);
  const int n_above = min(ctrl[t * kCtrlWords + kCtrlAbove], K);
  const int nc = ctrl[t * kCtrlWords + kCtrlCand];
  const int b1 = ctrl[t * kCtrlWords + kCtrlB1];
  int32_t* out = idx + (int64_t)t * k;
  const uint2* cl = cand + (int64_t)t * cand_stride;
  const int need = K - n_above;

  uint32_t tau = 0xffffffffu, pcut = 0u;  // nothing from the candidates by default
  if (need > 0 && nc > 0 && b1 >= 0) {
    // second digit (key bits 20..10) from the collect pass's histogram
    for (int i = threadIdx.x; i < kTopkBins; i += kFinalThreads)
      h[i] = hist2[(int64_t)t * kTopkBins + i];
    __syncthreads();
    find_cut(h, kTopkBins, (uint32_t)need, &s_bin, &s_above, scan);
    const int b2 = s_bin;
    const uint32_t need2 = (uint32_t)need - s_above;
    // third digit (bits 9..0) over the candidates in (b1, b2)
    for (int i = threadIdx.x; i < 1024; i += kFinalThreads) h[i] = 0u;
    __syncthreads();
    for_each_cand(cl, nc, [&](uint2 c) {
      if (((c.x >> 10) & (kTopkBins - 1)) == (uint32_t)b2) atomicAdd(&h[c.x & 1023u], 1u);
    });
    __syncthreads();
    find_cut(h, 1024, need2, &s_bin, &s_above, scan);
    const int b3 = s_bin;
    const uint32_t need3 = need2 - s_above;
    const uint32_t cnt_eq = h[b3];
    tau = ((uint32_t)b1 << 21) | ((uint32_t)b2 << 10) | (uint32_t)b3;
    pcut = 0xffffffffu;
    __syncthreads();
    if (need3 < cnt_eq) {
      // keep the need3 lowest positions among keys equal to tau: the need3
      // largest values of ~position
      uint32_t gt2 = 0;
      const uint32_t t_ = tau;
      const uint32_t npos = radix_select(
          nc, need3,
          [&](int i, uint32_t* x) {
            const uint2 c = cl[i];
            *x = ~c.y;
            return c.x == t_;
          },
          h, scan, &s_bin, &s_above, &gt2);
      pcut = ~npos;
    }
  }
  auto picked = [&](uint2 c) { return c.x > tau || (c.x == tau && c.y <= pcut); };

  if (v <= kBitmapWords * 32) {
    const int nwords = (v + 31) >> 5;
    for (int i = threadIdx.x; i < nwords; i += kFinalThreads) bitmap[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n_above; i += kFinalThreads) {
      const int s = out[i];
      atomicOr(&bitmap[s >> 5], 1u << (s & 31));
    }
    if (tau != 0xffffffffu || pcut != 0u) {
      for_each_cand(cl, nc, [&](uint2 c) {
        if (picked(c)) atomicOr(&bitmap[c.y >> 5], 1u << (c.y & 31));
      });
    }
    __syncthreads();
    // ascending compaction: thread i owns words [i*per, (i+1)*per)
    const int per = (nwords + kFinalThreads - 1) / kFinalThreads;
    const int w0 = threadIdx.x * per, w1 = min(nwords, w0 + per);
    uint32_t cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(bitmap[w]);
    uint32_t total;
    uint32_t at = block_exclusive_sum(cnt, wsum, &total);
    for (int w = w0; w < w1; ++w) {
      uint32_t m = bitmap[w];
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1;
        if (at < (uint32_t)K) out[at] = index_in_space(b, bi, space, kv_off, (w << 5) + bit);
        ++at;
      }
    }
    __syncthreads();
    for (int i = (int)min(total, (uint32_t)K) + threadIdx.x; i < k; i += kFinalThreads) out[i] = -1;
    return;
  }

  // long rows: gather into LDS and sort (K <= kSortCap)
  for (int i = threadIdx.x; i < n_above; i += kFinalThreads) sel[i] = out[i];
  if (threadIdx.x == 0) s_count = n_above;
  __syncthreads();
  if (tau != 0xffffffffu || pcut != 0u) {
    for_each_cand(cl, nc, [&](uint2 c) {
      if (picked(c)) {
        const int a = atomicAdd(&s_count, 1);
        if (a < kSortCap) sel[a] = (int32_t)c.y;
      }
    });
  }
  __syncthreads();
  int n2 = 1;
  while (n2 < K) n2 <<= 1;
  for (int i = K + threadIdx.x; i < n2; i += kFinalThreads) sel[i] = 0x7fffffff;
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n2 >> 1); i += kFinalThreads) {
        const int pos = 2 * i - (i & (stride - 1));
        const int par = pos + stride;
        const bool asc = (pos & size) == 0;
        const int a = sel[pos], c = sel[par];
        if ((a > c) == asc) {
          sel[pos] = c;
          sel[par] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < k; i += kFinalThreads)
    out[i] = i < K ? index_in_space(b, bi, space, kv_off, sel[i]) : -1;
}

// the selection of rows whose visible tokens all fit in k: every position
__global__ void select_all_kernel(BatchArgs b, int k, int32_t* __restrict__ idx) {
  const int t = blockIdx.y;
  const int v = row_len(b, t);
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < k; j += gridDim.x * blockDim.x)
    idx[(int64_t)t * k + j] = j < v ? j : -1;
}

}  // namespace

TopkWs topk_ws_layout(const BatchArgs& b) {
  TopkWs w;
  size_t off = 0;
  w.hist_off = off;  // hist1 then hist2, [T][2048] each
  off = align_up(off + (size_t)b.T * kTopkBins * 4 * 2, 256);
  w.ctrl_off = off;
  off = align_up(off + (size_t)b.T * kCtrlWords * 4, 256);
  w.cand_off = off;
  off = align_up(off + (size_t)b.T * (size_t)b.max_seqlen_k * 8, 256);
  w.total = off;
  return w;
}

bool topk_supported(const BatchArgs& b, int k) {
  // rows longer than the bitmap are sorted in LDS, which holds kSortCap
  return (int64_t)b.max_seqlen_k <= (int64_t)kBitmapWords * 32 || k <= kSortCap;
}

uint32_t* topk_hist1(const BatchArgs& b, void* ws) {
  return reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + topk_ws_layout(b).hist_off);
}

hipError_t launch_topk_zero(const BatchArgs& b, void* ws, hipStream_t s) {
  if (b.T == 0) return hipSuccess;
  const TopkWs L = topk_ws_layout(b);
  // histograms and control words start at zero (a fill kernel, not a
  // memset, so the sequence can be captured in a graph)
  const int64_t nz = (int64_t)(L.cand_off / 4);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)std::min<int64_t>((nz + 255) / 256, 4096)),
                     dim3(256), 0, s, static_cast<uint32_t*>(ws), nz);
  return hipGetLastError();
}

hipError_t launch_topk_select(const BatchArgs& b, const float* scores, int64_t ld, int k,
                              int32_t* idx, void* ws, hipStream_t s, int space,
                              const int32_t* kv_off) {
  if (b.T == 0) return hipSuccess;
  const TopkWs L = topk_ws_layout(b);
  char* base = static_cast<char*>(ws);
  uint32_t* hist1 = reinterpret_cast<uint32_t*>(base + L.hist_off);
  uint32_t* hist2 = hist1 + (size_t)b.T * kTopkBins;
  int32_t* ctrl = reinterpret_cast<int32_t*>(base + L.ctrl_off);
  uint2* cand = reinterpret_cast<uint2*>(base + L.cand_off);
  const int segs = std::max(1, (b.max_seqlen_k + kTopkSeg - 1) / kTopkSeg);
  dim3 g2(b.T, segs);
  hipLaunchKernelGGL(topk_collect_kernel, g2, dim3(kCollectThreads), 0, s, b, scores, ld, k, hist1,
                     ctrl, idx, cand, (int64_t)b.max_seqlen_k, hist2);
  hipLaunchKernelGGL(topk_final_kernel, dim3(b.T), dim3(kFinalThreads), 0, s, b, k, ctrl, hist2,
                     idx, cand, (int64_t)b.max_seqlen_k, space, kv_off);
  return hipGetLastError();
}

hipError_t launch_topk(const BatchArgs& b, const float* scores, int64_t ld, int k, int32_t* idx,
                       void* ws, hipStream_t s, int space, const int32_t* kv_off) {
  if (b.T == 0) return hipSuccess;
  hipError_t e = launch_topk_zero(b, ws, s);
  if (e != hipSuccess) return e;
  const int segs = std::max(1, (b.max_seqlen_k + kTopkSeg - 1) / kTopkSeg);
  hipLaunchKernelGGL(topk_hist_kernel, dim3(b.T, segs), dim3(kHistThreads), 0, s, b, scores, ld, k,
                     topk_hist1(b, ws));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_select(b, scores, ld, k, idx, ws, s, space, kv_off);
}

hipError_t launch_select_all(const BatchArgs& b, int k, int32_t* idx, hipStream_t s) {
  if (b.T == 0) return hipSuccess;
  hipLaunchKernelGGL(select_all_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)b.T), dim3(256), 0,
                     s, b, k, idx);
  return hipGetLastError();
}

}  // namespace dsa
