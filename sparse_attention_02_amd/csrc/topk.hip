// Per-row top-k for gfx950: radix select on order-preserving uint32 keys.
//
// Each row keeps the K = min(k, v_t) visible positions with the largest
// scores; at the k-th score ties go to the lower position ("MTP and sparse
// attention: NSA and DSA", DSA bullet: each query keeps its top 2048).
//
//   1. hist1   per-row histogram of the top 11 key bits (LDS histograms added
//              into global memory).  The fused decode step builds it inside
//              the indexer scan instead (no extra pass over the scores).
//   2. collect (row x 4096-score segment): each work-group finds the bin b1
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
#include <type_traits>

#include "device_common.h"

namespace dsa {
namespace {

constexpr int kHistThreads = 256;
constexpr int kCollectThreads = 256;
#ifndef DSA_COLLECT_SEG
#define DSA_COLLECT_SEG 4096
#endif
constexpr int kCollectSeg = DSA_COLLECT_SEG;                // scores per collect work-group
constexpr int kPerThread = kCollectSeg / kCollectThreads;   // scores per thread
static_assert(kPerThread <= 64 && kCollectSeg < 65536, "masks of 64 bits, 16-bit counts");
// bit masks over a thread's scores
using SegMask = std::conditional_t<(kPerThread > 32), uint64_t, uint32_t>;
constexpr int kFinalThreads = 1024;
constexpr int kBitmapWords = 12288;  // 48 KB: rows up to 393216 positions
constexpr int kSortCap = 4096;       // bitonic fallback (rows longer than the bitmap)
constexpr int kCandStage = 6144;     // candidates the final pass stages in LDS (48 KB)

// ctrl words per row
constexpr int kCtrlB1 = 0;     // threshold bin (-1: every visible position selected)
constexpr int kCtrlAbove = 1;  // positions written as "above"
constexpr int kCtrlCand = 2;   // candidates appended
constexpr int kCtrlWords = 4;

// p 16-byte aligned, n16 16-byte words
__global__ void zero_kernel(uint4* __restrict__ p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// a key that float_key made from a NaN (above +inf's key, or below -inf's)
__device__ __forceinline__ bool key_is_nan(uint32_t k) {
  return k > 0xff800000u || k < 0x007fffffu;
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
      if (base + (int)threadIdx.x + u * kHistThreads < s1) {
        device_check(b, key_is_nan(kk[u]), DSA_CHECK_NAN_SCORE);
        atomicAdd(&h[kk[u] >> 21], 1u);
      }
  }
  __syncthreads();
  uint32_t* gh = hist + (int64_t)t * kTopkBins;
  for (int i = threadIdx.x; i < kTopkBins; i += kHistThreads)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// Largest bin `bin` of h[0..nbins) with sum_{b > bin} h[b] < need <=
// sum_{b >= bin} h[b]; *above = sum_{b > bin} h[b].  Block-wide (blockDim.x a
// multiple of 64, at most 1024); need >= 1 and sum h >= need, else *bin is
// left as it was.  Each thread sums a run of bins, the suffix sums run as
// shuffles inside each wave plus one exchange of the wave totals through
// `scan` (at least 16 words of LDS): two barriers per call.
__device__ void find_cut(const uint32_t* h, int nbins, uint32_t need, int* bin, uint32_t* above,
                         uint32_t* scan) {
  const int nt = blockDim.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = nt >> 6;
  const int per = (nbins + nt - 1) / nt;
  const int lo = min(nbins, (int)threadIdx.x * per);
  const int hi = min(nbins, lo + per);
  uint32_t mine = 0;
  for (int i = lo; i < hi; ++i) mine += h[i];
  uint32_t inc = mine;  // inclusive suffix sum over the wave's lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(inc, off);
    if (lane + off < 64) inc += y;
  }
  if (lane == 0) scan[wave] = inc;
  __syncthreads();
  uint32_t run = inc - mine;  // sum of bins above this thread's range
  for (int w = wave + 1; w < nw; ++w) run += scan[w];
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

// VEC: rows 16-byte aligned with ld % 4 == 0, so element 4q + e of a thread
// is position s0 + 4 tid + 1024 q + e, read in 16-byte loads; else element
// j is position s0 + tid + 256 j, read one by one.  Which segment position a
// thread holds changes only the order of the appends, not the selection.
template <bool VEC>
__global__ __launch_bounds__(kCollectThreads) void topk_collect_kernel(
    BatchArgs b, const float* __restrict__ scores, int64_t ld, int k,
    const uint32_t* __restrict__ hist1, int32_t* __restrict__ ctrl, int32_t* __restrict__ idx,
    uint2* __restrict__ cand, int64_t cand_stride, uint32_t* __restrict__ hist2) {
  __shared__ __attribute__((aligned(16))) uint32_t h1[kTopkBins];
  __shared__ uint32_t h2[kTopkBins];
  __shared__ uint32_t scan[kCollectThreads];
  __shared__ uint32_t wsum[16];
  __shared__ uint32_t s_base[2];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  const int t = blockIdx.x;
  const int v = row_len(b, t);
  const int s0 = blockIdx.y * kCollectSeg;
  if (s0 >= v) return;
  const float* row = scores + (int64_t)t * ld;
  const bool all = v <= k;  // every visible position is selected

  // the row's first-digit histogram (8 bins per thread, two 16-byte loads),
  // then the segment's scores (coalesced loads, all issued before any is
  // used: positions past the row re-read its last score or group and are
  // masked below).  The threshold search below runs while the score loads
  // are in flight.
  constexpr int kHistPer = kTopkBins / kCollectThreads;
  static_assert(kHistPer == 8, "two 16-byte histogram loads per thread");
  uint4 hv[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
  if (!all) {
    const uint4* hp = reinterpret_cast<const uint4*>(hist1 + (int64_t)t * kTopkBins);
    hv[0] = hp[threadIdx.x];
    hv[1] = hp[threadIdx.x + kCollectThreads];
  }
  // position of element j of this thread
  auto pos_of = [&](int j) {
    return VEC ? s0 + 4 * (int)threadIdx.x + kCollectThreads * 4 * (j >> 2) + (j & 3)
               : s0 + (int)threadIdx.x + j * kCollectThreads;
  };
  uint32_t key[kPerThread];
  if (VEC) {
    const int last = (v - 1) & ~3;  // first position of the row's last 16-byte group
#pragma unroll
    for (int q = 0; q < kPerThread / 4; ++q) {
      const float4 x = *reinterpret_cast<const float4*>(
          row + min(s0 + 4 * (int)threadIdx.x + kCollectThreads * 4 * q, last));
      key[4 * q] = float_key(x.x);
      key[4 * q + 1] = float_key(x.y);
      key[4 * q + 2] = float_key(x.z);
      key[4 * q + 3] = float_key(x.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) key[j] = float_key(row[min(pos_of(j), v - 1)]);
  }
  reinterpret_cast<uint4*>(h1)[threadIdx.x] = hv[0];
  reinterpret_cast<uint4*>(h1)[threadIdx.x + kCollectThreads] = hv[1];
#pragma unroll
  for (int i = 0; i < kHistPer; ++i) h2[threadIdx.x + i * kCollectThreads] = 0u;
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
  SegMask am = 0, em = 0;  // bit j: element j is above / a candidate
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int s = pos_of(j);
    const int d = (int)(key[j] >> 21);
    if (s < v) {
      device_check(b, key_is_nan(key[j]), DSA_CHECK_NAN_SCORE);
      if (b1 < 0 || d > b1) am |= (SegMask)1 << j;
      else if (d == b1) em |= (SegMask)1 << j;
    }
  }
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if ((em >> j) & 1) atomicAdd(&h2[(key[j] >> 10) & (kTopkBins - 1)], 1u);

  // both counts in one scan: at most kCollectSeg (4096) per work-group, so 16 bits each
  uint32_t tot;
  const uint32_t ex = block_exclusive_sum(((uint32_t)__popcll(am) << 16) | (uint32_t)__popcll(em),
                                          wsum, &tot);
  const uint32_t ex_a = ex >> 16, ex_e = ex & 0xffffu;
  const uint32_t tot_a = tot >> 16, tot_e = tot & 0xffffu;
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
    const int s = pos_of(j);
    if ((am >> j) & 1) {
      if (ra + na < (uint32_t)k) out[ra + na] = s;
      ++na;
    }
    if ((em >> j) & 1) cl[ne++] = make_uint2(key[j], (uint32_t)s);
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
  __shared__ uint2 lcand[kCandStage];
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
  const bool refine = need > 0 && nc > 0 && b1 >= 0;
  const bool bitmap_form = v <= kBitmapWords * 32;

  // Everything the row needs from global memory is requested at once: the
  // second-digit histogram, the candidates (staged in LDS when they fit) and
  // the positions already selected as "above" (k <= 8192: at most 8 per
  // thread), so the work below waits for one round trip instead of one per
  // pass.
  constexpr int kAbovePer = DSA_MAX_TOPK / kFinalThreads;
  int32_t ab[kAbovePer];
#pragma unroll
  for (int j = 0; j < kAbovePer; ++j) {
    const int i = threadIdx.x + j * kFinalThreads;
    ab[j] = i < n_above ? out[i] : -1;
  }
  const bool staged = nc <= kCandStage;
  if (refine) {
    for (int i = threadIdx.x; i < kTopkBins; i += kFinalThreads)
      h[i] = hist2[(int64_t)t * kTopkBins + i];
    if (staged) {
      for (int base = 0; base < nc; base += 8 * kFinalThreads) {
        uint2 c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = cl[min(base + (int)threadIdx.x + u * kFinalThreads, nc - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (base + (int)threadIdx.x + u * kFinalThreads < nc)
            lcand[base + threadIdx.x + u * kFinalThreads] = c[u];
      }
    }
  }
  if (bitmap_form) {
    for (int i = threadIdx.x; i < ((v + 31) >> 5); i += kFinalThreads) bitmap[i] = 0u;
  }
  __syncthreads();
  // candidate i, from LDS or (more than kCandStage of them) from global memory
  auto cget = [&](int i) { return staged ? lcand[i] : cl[i]; };
  auto each_cand = [&](auto f) {
    if (staged) {
      for (int i = threadIdx.x; i < nc; i += kFinalThreads) f(lcand[i]);
    } else {
      for_each_cand(cl, nc, f);
    }
  };

  uint32_t tau = 0xffffffffu, pcut = 0u;  // nothing from the candidates by default
  if (refine) {
    // second digit (key bits 20..10) from the collect pass's histogram
    find_cut(h, kTopkBins, (uint32_t)need, &s_bin, &s_above, scan);
    const int b2 = s_bin;
    const uint32_t need2 = (uint32_t)need - s_above;
    // third digit (bits 9..0) over the candidates in (b1, b2)
    for (int i = threadIdx.x; i < 1024; i += kFinalThreads) h[i] = 0u;
    __syncthreads();
    each_cand([&](uint2 c) {
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
            const uint2 c = cget(i);
            *x = ~c.y;
            return c.x == t_;
          },
          h, scan, &s_bin, &s_above, &gt2);
      pcut = ~npos;
    }
  }
  auto picked = [&](uint2 c) { return c.x > tau || (c.x == tau && c.y <= pcut); };
  const bool from_cand = tau != 0xffffffffu || pcut != 0u;

  if (bitmap_form) {
#pragma unroll
    for (int j = 0; j < kAbovePer; ++j)
      if (ab[j] >= 0) atomicOr(&bitmap[ab[j] >> 5], 1u << (ab[j] & 31));
    if (from_cand) {
      each_cand([&](uint2 c) {
        if (picked(c)) atomicOr(&bitmap[c.y >> 5], 1u << (c.y & 31));
      });
    }
    __syncthreads();
    // ascending compaction: thread i owns words [i*per, (i+1)*per)
    const int nwords = (v + 31) >> 5;
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
#pragma unroll
  for (int j = 0; j < kAbovePer; ++j)
    if (ab[j] >= 0) sel[threadIdx.x + j * kFinalThreads] = ab[j];
  if (threadIdx.x == 0) s_count = n_above;
  __syncthreads();
  if (from_cand) {
    each_cand([&](uint2 c) {
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

// ---- rows of at most 65536 positions: one work-group per row -------------
//
// The row's keys stay in registers (KPT per thread, read once with 16-byte
// loads) and the three radix passes (11, 11, 10 bits) histogram them in LDS,
// so the selection needs one read of the scores and no global atomics,
// candidate lists or second launch.  Keys equal to the threshold are ranked
// by position through an LDS bitmap (the lowest positions win), and the
// selected positions leave in ascending order by a compaction of the bitmap.

constexpr int kRowThreads = 1024;
constexpr int kRowMax = 64 * kRowThreads;  // longest row: 64 keys per thread
constexpr int kCopies = 8;                 // copies of the pass-1 histogram
constexpr int kCopyStride = kTopkBins + 1;

template <int KPT>
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(
    BatchArgs b, const float* __restrict__ scores, int64_t ld, int k, int32_t* __restrict__ idx,
    int space, const int32_t* __restrict__ kv_off) {
  constexpr int Q = KPT / 4;                // 16-byte groups per thread
  constexpr int NW = KPT * kRowThreads / 32;  // bitmap words
  // pass-1 histogram in kCopies copies (lane l counts into copy l % kCopies,
  // the copies a bank apart): a row's keys crowd into the few first-digit
  // bins of their binades, and same-bin increments from one instruction
  // serialise unless spread over copies
  __shared__ uint32_t hc[kCopies * kCopyStride];
  __shared__ uint32_t h[kTopkBins];
  __shared__ uint32_t bm[NW];   // selected positions
  __shared__ uint32_t tie[NW];  // positions whose key equals the threshold
  __shared__ uint32_t wsum[16];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  const int t = blockIdx.x;
  const int bi = row_request(b.cu, b.B, t);
  const int v = row_visible(b, bi, t);
  const int K = min(k, v);
  const int tid = threadIdx.x;
  int32_t* out = idx + (int64_t)t * k;
  if (v <= k) {
    // every visible position is selected
    for (int i = tid; i < k; i += kRowThreads)
      out[i] = i < v ? index_in_space(b, bi, space, kv_off, i) : -1;
    return;
  }

  // group q of this thread: positions 4 tid + 4096 q + e, e < 4 (groups past
  // the row re-read its last aligned group and are masked below)
  const float* row = scores + (int64_t)t * ld;
  const int last = (v - 1) & ~3;
  v4f x[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q)
    x[q] = *reinterpret_cast<const v4f*>(row + min(4 * tid + 4096 * q, last));
  uint32_t key[Q][4];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) key[q][e] = float_key(x[q][e]);
  auto valid = [&](int q, int e) { return 4 * tid + 4096 * q + e < v; };

  // pass 1: bits 31..21
  for (int i = tid; i < kCopies * kCopyStride; i += kRowThreads) hc[i] = 0u;
  __syncthreads();
  {
    uint32_t* mine = hc + (tid % kCopies) * kCopyStride;
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (valid(q, e)) {
          device_check(b, key_is_nan(key[q][e]), DSA_CHECK_NAN_SCORE);
          atomicAdd(&mine[key[q][e] >> 21], 1u);
        }
  }
  __syncthreads();
  for (int i = tid; i < kTopkBins; i += kRowThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < kCopies; ++j) c += hc[j * kCopyStride + i];
    h[i] = c;
  }
  __syncthreads();
  if (tid == 0) s_bin = 0;
  find_cut(h, kTopkBins, (uint32_t)K, &s_bin, &s_above, wsum);
  const uint32_t b1 = (uint32_t)s_bin;
  uint32_t need = (uint32_t)K - s_above;
  __syncthreads();
  // pass 2: bits 20..10 of the keys in bin b1
  for (int i = tid; i < kTopkBins; i += kRowThreads) h[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (valid(q, e) && (key[q][e] >> 21) == b1) atomicAdd(&h[(key[q][e] >> 10) & 2047u], 1u);
  __syncthreads();
  if (tid == 0) s_bin = 0;
  find_cut(h, kTopkBins, need, &s_bin, &s_above, wsum);
  const uint32_t p2 = (b1 << 11) | (uint32_t)s_bin;
  need -= s_above;
  __syncthreads();
  // pass 3: bits 9..0 of the keys whose top 22 bits are p2
  for (int i = tid; i < 1024; i += kRowThreads) h[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (valid(q, e) && (key[q][e] >> 10) == p2) atomicAdd(&h[key[q][e] & 1023u], 1u);
  __syncthreads();
  if (tid == 0) s_bin = 0;
  find_cut(h, 1024, need, &s_bin, &s_above, wsum);
  const uint32_t tau = (p2 << 10) | (uint32_t)s_bin;
  const uint32_t need3 = need - s_above;  // keys equal to tau to keep (>= 1)
  const uint32_t cnt_eq = h[s_bin];

  // keys above tau, and keys equal to it, as bitmaps over the positions
  // (the 4 positions of a group share a word)
  for (int i = tid; i < NW; i += kRowThreads) {
    bm[i] = 0u;
    tie[i] = 0u;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!valid(q, e)) continue;
      if (key[q][e] > tau) gt |= 1u << e;
      else if (key[q][e] == tau) eq |= 1u << e;
    }
    const int word = (tid >> 3) + 128 * q;
    const int sh = 4 * (tid & 7);
    if (gt) atomicOr(&bm[word], gt << sh);
    if (eq) atomicOr(&tie[word], eq << sh);
  }
  __syncthreads();
  // thread i owns words [i*per, (i+1)*per)
  constexpr int per = (NW + kRowThreads - 1) / kRowThreads;
  const int w0 = min(NW, tid * per), w1 = min(NW, w0 + per);
  if (need3 < cnt_eq) {
    // the need3 lowest tie positions: ranks from a prefix sum in word order
    uint32_t cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(tie[w]);
    uint32_t tot;
    uint32_t at = block_exclusive_sum(cnt, wsum, &tot);
    for (int w = w0; w < w1; ++w) {
      uint32_t m = tie[w], keep = 0;
      while (m) {
        const uint32_t bit = m & (0u - m);
        m ^= bit;
        if (at < need3) keep |= bit;
        ++at;
      }
      bm[w] |= keep;
    }
  } else {
    for (int w = w0; w < w1; ++w) bm[w] |= tie[w];
  }
  __syncthreads();
  // ascending compaction
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  uint32_t total;
  uint32_t at = block_exclusive_sum(cnt, wsum, &total);
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bm[w];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      if (at < (uint32_t)K) out[at] = index_in_space(b, bi, space, kv_off, (w << 5) + bit);
      ++at;
    }
  }
  for (int i = K + tid; i < k; i += kRowThreads) out[i] = -1;
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
  // (cand_off is a multiple of 256 bytes and ws 16-byte aligned)
  const int64_t nz = (int64_t)(L.cand_off / 16);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)std::min<int64_t>((nz + 255) / 256, 1024)),
                     dim3(256), 0, s, static_cast<uint4*>(ws), nz);
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
  const int segs = std::max(1, (b.max_seqlen_k + kCollectSeg - 1) / kCollectSeg);
  dim3 g2(b.T, segs);
  if ((reinterpret_cast<uintptr_t>(scores) & 15) == 0 && ld % 4 == 0)
    hipLaunchKernelGGL(topk_collect_kernel<true>, g2, dim3(kCollectThreads), 0, s, b, scores, ld, k,
                       hist1, ctrl, idx, cand, (int64_t)b.max_seqlen_k, hist2);
  else
    hipLaunchKernelGGL(topk_collect_kernel<false>, g2, dim3(kCollectThreads), 0, s, b, scores, ld,
                       k, hist1, ctrl, idx, cand, (int64_t)b.max_seqlen_k, hist2);
  hipLaunchKernelGGL(topk_final_kernel, dim3(b.T), dim3(kFinalThreads), 0, s, b, k, ctrl, hist2,
                     idx, cand, (int64_t)b.max_seqlen_k, space, kv_off);
  return hipGetLastError();
}

hipError_t launch_topk(const BatchArgs& b, const float* scores, int64_t ld, int k, int32_t* idx,
                       void* ws, hipStream_t s, int space, const int32_t* kv_off) {
  if (b.T == 0) return hipSuccess;
  if (topk_rows_fit(b, scores, ld)) return launch_topk_rows(b, scores, ld, k, idx, s, space, kv_off);
  hipError_t e = launch_topk_zero(b, ws, s);
  if (e != hipSuccess) return e;
  const int segs = std::max(1, (b.max_seqlen_k + kTopkSeg - 1) / kTopkSeg);
  hipLaunchKernelGGL(topk_hist_kernel, dim3(b.T, segs), dim3(kHistThreads), 0, s, b, scores, ld, k,
                     topk_hist1(b, ws));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_select(b, scores, ld, k, idx, ws, s, space, kv_off);
}

bool topk_rows_fit(const BatchArgs& b, const float* scores, int64_t ld) {
  return b.max_seqlen_k <= kRowMax && (reinterpret_cast<uintptr_t>(scores) & 15) == 0 &&
         ld % 4 == 0;
}

hipError_t launch_topk_rows(const BatchArgs& b, const float* scores, int64_t ld, int k,
                            int32_t* idx, hipStream_t s, int space, const int32_t* kv_off) {
  if (b.T == 0) return hipSuccess;
  const dim3 grid(b.T), block(kRowThreads);
  if (b.max_seqlen_k <= 8 * kRowThreads)
    hipLaunchKernelGGL(topk_row_kernel<8>, grid, block, 0, s, b, scores, ld, k, idx, space, kv_off);
  else if (b.max_seqlen_k <= 32 * kRowThreads)
    hipLaunchKernelGGL(topk_row_kernel<32>, grid, block, 0, s, b, scores, ld, k, idx, space, kv_off);
  else
    hipLaunchKernelGGL(topk_row_kernel<64>, grid, block, 0, s, b, scores, ld, k, idx, space, kv_off);
  return hipGetLastError();
}

hipError_t launch_select_all(const BatchArgs& b, int k, int32_t* idx, hipStream_t s) {
  if (b.T == 0) return hipSuccess;
  hipLaunchKernelGGL(select_all_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)b.T), dim3(256), 0,
                     s, b, k, idx);
  return hipGetLastError();
}

}  // namespace dsa
