// Per-row top-k for gfx950: radix select on order-preserving uint32 keys.
//
// Each row keeps the K = min(k, v_t) visible positions with the largest
// scores; at the k-th score ties go to the lower position ("MTP and sparse
// attention: NSA and DSA", DSA bullet: each query keeps its top 2048).
//
//   1. hist     (row x segment): LDS histogram of the top 11 key bits,
//               added into a per-row global histogram.
//   2. thresh   (row): the bin b1 holding the K-th largest key.
//   3. collect  (row x segment): keys in bins above b1 are selected
//               outright; keys in b1 are appended to a candidate list.
//               Appends use one atomic per wave (ballot + mbcnt ranks).
//   4. final    (row): exact radix select of the remaining count among the
//               candidates (three 11/11/10-bit passes over the full key),
//               ties at the threshold resolved by a second radix select on
//               the position (lowest positions win), then the K positions
//               are sorted ascending in LDS and written with -1 padding.
// Output is therefore deterministic: the selected set, ascending.
#include "device_common.h"

namespace dsa {
namespace {

constexpr int kHistThreads = 256;
constexpr int kFinalThreads = 1024;

// ctrl words per row
constexpr int kCtrlB1 = 0;      // threshold bin (-1: every visible position selected)
constexpr int kCtrlAbove = 1;   // positions written so far as "above"
constexpr int kCtrlCand = 2;    // candidates appended so far
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
  for (int s = s0 + threadIdx.x; s < s1; s += kHistThreads)
    atomicAdd(&h[float_key(row[s]) >> 21], 1u);
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

__global__ __launch_bounds__(kHistThreads) void topk_thresh_kernel(BatchArgs b, int k,
                                                                    const uint32_t* __restrict__ hist,
                                                                    int32_t* __restrict__ ctrl) {
  __shared__ uint32_t h[kTopkBins];
  __shared__ uint32_t scan[kHistThreads];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  const int t = blockIdx.x;
  const int v = row_len(b, t);
  if (v <= k) {
    if (threadIdx.x == 0) ctrl[t * kCtrlWords + kCtrlB1] = -1;
    return;
  }
  for (int i = threadIdx.x; i < kTopkBins; i += kHistThreads) h[i] = hist[(int64_t)t * kTopkBins + i];
  __syncthreads();
  find_cut(h, kTopkBins, (uint32_t)k, &s_bin, &s_above, scan);
  if (threadIdx.x == 0) ctrl[t * kCtrlWords + kCtrlB1] = s_bin;
}

// Appends the lanes whose pred is set to list at ranks taken from one
// atomic counter per wave; returns nothing.  Order among lanes follows the
// lane index; order among waves follows the atomics.
template <typename T>
__device__ __forceinline__ void wave_append(bool pred, T value, T* list, int32_t* counter) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0) return;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((long long)mask) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(counter, __popcll(mask));
  base = __shfl(base, leader);
  if (pred) {
    const uint64_t below = lane ? (mask & ((~0ull) >> (64 - lane))) : 0ull;
    list[base + __popcll(below)] = value;
  }
}

__global__ __launch_bounds__(kHistThreads) void topk_collect_kernel(
    BatchArgs b, const float* __restrict__ scores, int64_t ld, int k, int32_t* __restrict__ ctrl,
    int32_t* __restrict__ idx, uint2* __restrict__ cand, int64_t cand_stride) {
  const int t = blockIdx.x;
  const int v = row_len(b, t);
  const int s0 = blockIdx.y * kTopkSeg;
  if (s0 >= v) return;
  const int s1 = min(v, s0 + kTopkSeg);
  const int b1 = ctrl[t * kCtrlWords + kCtrlB1];
  const float* row = scores + (int64_t)t * ld;
  int32_t* out = idx + (int64_t)t * k;
  uint2* cl = cand + (int64_t)t * cand_stride;
  // every lane of a wave runs the same number of iterations (ballots)
  for (int base = s0; base < s1; base += kHistThreads) {
    const int s = base + threadIdx.x;
    const bool in = s < s1;
    const uint32_t key = in ? float_key(row[s]) : 0u;
    const int d = (int)(key >> 21);
    const bool above = in && (b1 < 0 || d > b1);
    const bool eq = in && b1 >= 0 && d == b1;
    wave_append<int32_t>(above, s, out, &ctrl[t * kCtrlWords + kCtrlAbove]);
    wave_append<uint2>(eq, make_uint2(key, (uint32_t)s), cl, &ctrl[t * kCtrlWords + kCtrlCand]);
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
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      uint32_t x;
      if (!get(i, &x)) continue;
      if (hs < 32 && (x >> hs) != (prefix >> hs)) continue;
      atomicAdd(&h[(x >> sh) & (nb - 1)], 1u);
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

__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(BatchArgs b, int k,
                                                                  const int32_t* __restrict__ ctrl,
                                                                  int32_t* __restrict__ idx,
                                                                  const uint2* __restrict__ cand,
                                                                  int64_t cand_stride) {
  __shared__ int32_t sel[DSA_MAX_TOPK];
  __shared__ uint32_t h[kTopkBins];
  __shared__ uint32_t scan[kFinalThreads];
  __shared__ int s_bin;
  __shared__ uint32_t s_above;
  __shared__ int32_t s_count;
  const int t = blockIdx.x;
  const int v = row_len(b, t);
  const int K = min(k, v);
  const int n_above = ctrl[t * kCtrlWords + kCtrlAbove];
  const int nc = ctrl[t * kCtrlWords + kCtrlCand];
  int32_t* out = idx + (int64_t)t * k;
  const uint2* cl = cand + (int64_t)t * cand_stride;

  for (int i = threadIdx.x; i < n_above && i < K; i += kFinalThreads) sel[i] = out[i];
  if (threadIdx.x == 0) s_count = min(n_above, K);
  __syncthreads();

  const int need = K - n_above;
  if (need > 0 && nc > 0) {
    uint32_t gt = 0;
    const uint32_t tau = radix_select(
        nc, (uint32_t)need,
        [&](int i, uint32_t* x) {
          *x = cl[i].x;
          return true;
        },
        h, scan, &s_bin, &s_above, &gt);
    const uint32_t need_eq = (uint32_t)need - gt;
    // among keys equal to tau keep the need_eq lowest positions:
    // radix-select the need_eq largest of ~pos
    uint32_t gt2 = 0;
    const uint32_t npos = radix_select(
        nc, need_eq,
        [&](int i, uint32_t* x) {
          const uint2 c = cl[i];
          *x = ~c.y;
          return c.x == tau;
        },
        h, scan, &s_bin, &s_above, &gt2);
    const uint32_t pcut = ~npos;  // positions <= pcut among ties are kept
    for (int i = threadIdx.x; i < nc; i += kFinalThreads) {
      const uint2 c = cl[i];
      if (c.x > tau || (c.x == tau && c.y <= pcut)) {
        const int at = atomicAdd(&s_count, 1);
        if (at < DSA_MAX_TOPK) sel[at] = (int32_t)c.y;
      }
    }
    __syncthreads();
  }

  // bitonic sort of sel[0..K) ascending (padding with INT_MAX)
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
  for (int i = threadIdx.x; i < k; i += kFinalThreads) out[i] = i < K ? sel[i] : -1;
}

}  // namespace

TopkWs topk_ws_layout(const BatchArgs& b) {
  TopkWs w;
  size_t off = 0;
  w.hist_off = off;
  off = align_up(off + (size_t)b.T * kTopkBins * 4, 256);
  w.ctrl_off = off;
  off = align_up(off + (size_t)b.T * kCtrlWords * 4, 256);
  w.cand_off = off;
  off = align_up(off + (size_t)b.T * (size_t)b.max_seqlen_k * 8, 256);
  w.total = off;
  return w;
}

hipError_t launch_topk(const BatchArgs& b, const float* scores, int64_t ld, int k, int32_t* idx,
                       void* ws, hipStream_t s) {
  if (b.T == 0) return hipSuccess;
  const TopkWs L = topk_ws_layout(b);
  char* base = static_cast<char*>(ws);
  uint32_t* hist = reinterpret_cast<uint32_t*>(base + L.hist_off);
  int32_t* ctrl = reinterpret_cast<int32_t*>(base + L.ctrl_off);
  uint2* cand = reinterpret_cast<uint2*>(base + L.cand_off);
  // histogram and control words start at zero (a fill kernel, not a memset,
  // so the sequence can be captured in a graph)
  const int64_t nz = (int64_t)(L.cand_off / 4);
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)std::min<int64_t>((nz + 255) / 256, 4096)),
                     dim3(256), 0, s, reinterpret_cast<uint32_t*>(base), nz);
  const int segs = std::max(1, (b.max_seqlen_k + kTopkSeg - 1) / kTopkSeg);
  dim3 g2(b.T, segs);
  hipLaunchKernelGGL(topk_hist_kernel, g2, dim3(kHistThreads), 0, s, b, scores, ld, k, hist);
  hipLaunchKernelGGL(topk_thresh_kernel, dim3(b.T), dim3(kHistThreads), 0, s, b, k, hist, ctrl);
  hipLaunchKernelGGL(topk_collect_kernel, g2, dim3(kHistThreads), 0, s, b, scores, ld, k, ctrl,
                     idx, cand, (int64_t)b.max_seqlen_k);
  hipLaunchKernelGGL(topk_final_kernel, dim3(b.T), dim3(kFinalThreads), 0, s, b, k, ctrl, idx,
                     cand, (int64_t)b.max_seqlen_k);
  return hipGetLastError();
}

}  // namespace dsa
