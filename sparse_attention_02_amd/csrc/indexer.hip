// Lightning-indexer scan for gfx950.
//
// I(t,s) = q_scale(t) * k_scale(s) * sum_h w(t,h) * max(0, q8(t,h) . k8(s))
// ("MTP and sparse attention: NSA and DSA", DSA bullet; the per-token scales
// are positive, so they factor out of the ReLU exactly).
//
// One work-group = one request x one group of RG query rows x one chunk of
// cache pages.  Each of its 4 waves owns 16 of the 64 tokens of a page.  The
// small dense contraction (RG*64 head rows x 16 keys x 128 dims) runs on
// v_mfma_f32_16x16x128_f8f6f4 with the queries held in registers for the
// whole chunk and the keys streamed straight from HBM into registers with
// two 16-byte loads per lane (no LDS).  The ReLU * w head reduction is an
// fp32 VALU epilogue: 4 heads in-lane per MFMA, then two cross-lane steps.
// The keys of a request are read once and shared by all its rows.
#include "device_common.h"

namespace dsa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8i load_frag(const uint8_t* p) {
  const v4i* s = reinterpret_cast<const v4i*>(p);
  v4i a = __builtin_nontemporal_load(s);
  v4i c = __builtin_nontemporal_load(s + 1);
  v8i r = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
  return r;
}

__device__ __forceinline__ v8i load_frag_cached(const uint8_t* p) {
  const uint4* s = reinterpret_cast<const uint4*>(p);
  uint4 a = s[0], c = s[1];
  v8i r = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)c.x, (int)c.y, (int)c.z, (int)c.w};
  return r;
}

// NT: keys are read by exactly one work-group (one row group per request),
// so they bypass the caches; otherwise several row groups re-read them.
template <int RG, bool NT>
__global__ __launch_bounds__(kThreads) void index_score_kernel(
    BatchArgs b, const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k8,
    const float* __restrict__ k_scale, float* __restrict__ scores, int64_t ld, int chunk_pages) {
  const int group = blockIdx.x;
  const int chunk = blockIdx.y;
  const int bi = blockIdx.z;
  const int c0 = b.cu[bi];
  const int n = b.cu[bi + 1] - c0;
  const int r0 = group * RG;
  if (r0 >= n) return;
  const int nr = min(RG, n - r0);
  const int L = clamp_len(b, b.lens[bi]);
  // the group's last row sees the most tokens
  const int vmax = min(L, max(0, L - n + 1 + r0 + nr - 1));
  const int p_begin = chunk * chunk_pages;
  const int p_end = min(p_begin + chunk_pages, (vmax + 63) >> 6);
  if (p_begin >= p_end) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15;  // key within the wave's 16
  const int g = lane >> 4;  // k-group of the operands / row group of the result

  // A operands: q8[t, 16m + j, 32g .. 32g+32) for each row r and head tile m.
  v8i qf[RG][4];
  float wr[RG][4][4];
  float qs[RG];
  int vis[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int t = c0 + r0 + min(r, nr - 1);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      qf[r][m] = load_frag_cached(q8 + ((int64_t)t * DSA_IDX_HEADS + 16 * m + j) * DSA_IDX_DIM +
                                  32 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[r][m][i] = w[(int64_t)t * DSA_IDX_HEADS + 16 * m + 4 * g + i];
    }
    qs[r] = q_scale[t];
    vis[r] = r < nr ? min(L, max(0, L - n + 1 + r0 + r)) : 0;
  }

  const int32_t* ptab = b.pages + (int64_t)bi * b.max_pages;
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  // software pipeline: keys of page p+1 load while page p computes
  int page = ptab[p_begin];
  bool ok = page >= 0 && page < b.num_pages;
  int64_t slot = (int64_t)(ok ? page : 0) * DSA_PAGE_SIZE + 16 * wave + j;
  v8i kf = NT ? load_frag(k8 + slot * DSA_IDX_DIM + 32 * g)
              : load_frag_cached(k8 + slot * DSA_IDX_DIM + 32 * g);
  float ks = k_scale[slot];

  for (int p = p_begin; p < p_end; ++p) {
    v8i kf_next = kf;
    float ks_next = ks;
    bool ok_next = false;
    if (p + 1 < p_end) {
      const int pg = ptab[p + 1];
      ok_next = pg >= 0 && pg < b.num_pages;
      const int64_t sl = (int64_t)(ok_next ? pg : 0) * DSA_PAGE_SIZE + 16 * wave + j;
      kf_next = NT ? load_frag(k8 + sl * DSA_IDX_DIM + 32 * g)
                   : load_frag_cached(k8 + sl * DSA_IDX_DIM + 32 * g);
      ks_next = k_scale[sl];
    }

    float sum[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      sum[r] = 0.f;
      if (r < nr) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          v4f acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[r][m], kf, zero, 0, 0, 0,
                                                                      0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) sum[r] = fmaf(wr[r][m][i], fmaxf(acc[i], 0.f), sum[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      sum[r] += __shfl_xor(sum[r], 16);
      sum[r] += __shfl_xor(sum[r], 32);
    }
    // lane group g stores row g of the group
    if (ok && g < nr) {
      float v = sum[0] * qs[0];
#pragma unroll
      for (int r = 1; r < RG; ++r)
        if (g == r) v = sum[r] * qs[r];
      int vg = vis[0];
#pragma unroll
      for (int r = 1; r < RG; ++r)
        if (g == r) vg = vis[r];
      const int s = p * DSA_PAGE_SIZE + 16 * wave + j;
      if (s < vg) scores[(int64_t)(c0 + r0 + g) * ld + s] = v * ks;
    }
    kf = kf_next;
    ks = ks_next;
    ok = ok_next;
  }
}

}  // namespace

hipError_t launch_index_score(const BatchArgs& b, const uint8_t* q8, const float* q_scale,
                              const float* w, const uint8_t* k8, const float* k_scale,
                              float* scores, int64_t ld, hipStream_t s) {
  if (b.B == 0 || b.T == 0 || b.max_seqlen_k == 0) return hipSuccess;
  const int rg = b.max_q <= 1 ? 1 : (b.max_q <= 2 ? 2 : 4);
  const int groups = (b.max_q + rg - 1) / rg;
  const int total_pages = (b.max_seqlen_k + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE;
  // chunk length: enough work-groups to fill the chip several times over,
  // at most 16 pages (1024 keys) per work-group
  int chunk_pages = 16;
  const long long want = 8LL * 256;
  while (chunk_pages > 2 &&
         (long long)b.B * groups * ((total_pages + chunk_pages - 1) / chunk_pages) < want)
    chunk_pages >>= 1;
  const int chunks = (total_pages + chunk_pages - 1) / chunk_pages;
  dim3 grid(groups, chunks, b.B);
  if (rg == 1)
    hipLaunchKernelGGL((index_score_kernel<1, true>), grid, dim3(kThreads), 0, s, b, q8, q_scale,
                       w, k8, k_scale, scores, ld, chunk_pages);
  else if (rg == 2)
    hipLaunchKernelGGL((index_score_kernel<2, true>), grid, dim3(kThreads), 0, s, b, q8, q_scale,
                       w, k8, k_scale, scores, ld, chunk_pages);
  else if (groups == 1)
    hipLaunchKernelGGL((index_score_kernel<4, true>), grid, dim3(kThreads), 0, s, b, q8, q_scale,
                       w, k8, k_scale, scores, ld, chunk_pages);
  else
    hipLaunchKernelGGL((index_score_kernel<4, false>), grid, dim3(kThreads), 0, s, b, q8,
                       q_scale, w, k8, k_scale, scores, ld, chunk_pages);
  return hipGetLastError();
}

}  // namespace dsa
