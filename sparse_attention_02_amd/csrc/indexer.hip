// Lightning-indexer scan for gfx950.
//
// I(t,s) = q_scale(t) * k_scale(s) * sum_h w(t,h) * max(0, q8(t,h) . k8(s))
// ("MTP and sparse attention: NSA and DSA", DSA bullet; the per-token scales
// are positive, so they factor out of the ReLU exactly).
//
// One work-group = one request x one group of RG query rows x one chunk of
// kChunk cache pages.  Each of its 4 waves owns 16 of the 64 tokens of a
// page.  The small dense contraction (RG*64 head rows x 16 keys x 128 dims)
// runs on v_mfma_f32_16x16x128_f8f6f4 with the queries held in registers for
// the whole chunk and the keys streamed straight from HBM into registers
// with two 16-byte loads per lane (no LDS).  The page loop is fully unrolled
// and branch-free (loads past the chunk's end re-read its last page and are
// not stored), NPF pages ahead of the math, so the compiler can wait on each
// page's own loads only and keep NPF pages in flight per wave.  The ReLU * w
// head reduction is an fp32 VALU epilogue: 4 heads in-lane per MFMA, then two
// cross-lane steps.  The keys of a request are read once and shared by all
// its rows.  With HIST the epilogue also counts each score's top-11-bit key
// digit into an LDS histogram per row, added to the row's global histogram
// at the end (the first radix pass of the top-k, without re-reading scores).
#include "device_common.h"

namespace dsa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 16;  // pages per work-group

typedef int v4i __attribute__((ext_vector_type(4)));

// max(x, 0) on the bit pattern: a non-negative float is a non-negative
// int32 and a negative one a negative int32, so one integer max is the ReLU
// (and needs no NaN quieting, unlike the float max)
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ v8i load_frag_nt(const uint8_t* p) {
  const v4i* s = reinterpret_cast<const v4i*>(p);
  v4i a = __builtin_nontemporal_load(s);
  v4i c = __builtin_nontemporal_load(s + 1);
  v8i r = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
  return r;
}

__device__ __forceinline__ v8i load_frag(const uint8_t* p) {
  const v4i* s = reinterpret_cast<const v4i*>(p);
  v4i a = s[0], c = s[1];
  v8i r = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
  return r;
}

// NT: keys are read by exactly one work-group (one row group per request),
// so they bypass the caches; otherwise several row groups re-read them.
template <int RG, int NPF, bool NT, bool HIST>
__global__ __launch_bounds__(kThreads) void index_score_kernel(
    BatchArgs b, const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k8,
    const float* __restrict__ k_scale, float* __restrict__ scores, int64_t ld,
    uint32_t* __restrict__ hist) {
  __shared__ uint32_t lh[HIST ? RG * kTopkBins : 1];
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
  const int p_begin = chunk * kChunk;
  const int p_end = min(p_begin + kChunk, (vmax + 63) >> 6);
  if (p_begin >= p_end) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15;  // key within the wave's 16
  const int g = lane >> 4;  // k-group of the operands / row of the result

  if (HIST) {
    for (int i = threadIdx.x; i < RG * kTopkBins; i += kThreads) lh[i] = 0u;
  }

  // page i of the chunk (past the end: the last page again; bad ids read
  // page 0 and are not stored)
  const int32_t* ptab = b.pages + (int64_t)bi * b.max_pages;
  const int lane_key = 16 * wave + j;
  auto page_id = [&](int i) { return ptab[min(p_begin + i, p_end - 1)]; };
  auto page_ok = [&](int pg) { return pg >= 0 && pg < b.num_pages; };
  auto key_ptr = [&](int pg) {
    return k8 + (int64_t)(page_ok(pg) ? pg : 0) * (DSA_PAGE_SIZE * DSA_IDX_DIM) +
           (lane_key * DSA_IDX_DIM + 32 * g);
  };
  auto scale_ptr = [&](int pg) {
    return k_scale + (int64_t)(page_ok(pg) ? pg : 0) * DSA_PAGE_SIZE + lane_key;
  };

  // key ring: NPF pages in flight
  v8i kf[NPF];
  float ksr[NPF];
#pragma unroll
  for (int u = 0; u < NPF; ++u) {
    const int pg = page_id(u);
    kf[u] = NT ? load_frag_nt(key_ptr(pg)) : load_frag(key_ptr(pg));
    ksr[u] = *scale_ptr(pg);
  }

  // A operands: q8[t, 16m + j, 32g .. 32g+32) for each row r and head tile m
  // (rows past the request's last repeat it; their results are not stored)
  v8i qf[RG][4];
  float wr[RG][4][4];
  float qs_g = 0.f;
  int vis_g = 0;
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int t = c0 + r0 + min(r, nr - 1);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      qf[r][m] = load_frag(q8 + ((int64_t)t * DSA_IDX_HEADS + 16 * m + j) * DSA_IDX_DIM + 32 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) wr[r][m][e] = w[(int64_t)t * DSA_IDX_HEADS + 16 * m + 4 * g + e];
    }
    if (g == r) {
      qs_g = q_scale[t];
      vis_g = r < nr ? min(L, max(0, L - n + 1 + r0 + r)) : 0;
    }
  }
  float* srow = scores + (int64_t)(c0 + r0 + min(g, nr - 1)) * ld;
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  if (HIST) __syncthreads();

#pragma unroll
  for (int i = 0; i < kChunk; ++i) {
    const v8i kcur = kf[i % NPF];
    const float kscur = ksr[i % NPF];
    if (i + NPF < kChunk) {
      const int pg = page_id(i + NPF);
      kf[i % NPF] = NT ? load_frag_nt(key_ptr(pg)) : load_frag(key_ptr(pg));
      ksr[i % NPF] = *scale_ptr(pg);
    }
    float sum[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      sum[r] = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const v4f acc =
            __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[r][m], kcur, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[r] = fmaf(wr[r][m][e], relu(acc[e]), sum[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      sum[r] += __shfl_xor(sum[r], 16);
      sum[r] += __shfl_xor(sum[r], 32);
    }
    float mine = sum[0];
#pragma unroll
    for (int r = 1; r < RG; ++r)
      if (g == r) mine = sum[r];
    const int s = (p_begin + i) * DSA_PAGE_SIZE + 16 * wave + j;
    if (page_ok(page_id(i)) && p_begin + i < p_end && g < nr && s < vis_g) {
      const float sc = mine * qs_g * kscur;
      srow[s] = sc;
      if (HIST) atomicAdd(&lh[g * kTopkBins + (float_key(sc) >> 21)], 1u);
    }
  }

  if (HIST) {
    __syncthreads();
    for (int i = threadIdx.x; i < nr * kTopkBins; i += kThreads) {
      const uint32_t c = lh[i];
      if (c) atomicAdd(&hist[(int64_t)(c0 + r0 + i / kTopkBins) * kTopkBins + (i % kTopkBins)], c);
    }
  }
}

template <int RG, int NPF, bool NT>
hipError_t launch_rg(dim3 grid, hipStream_t s, const BatchArgs& b, const uint8_t* q8,
                     const float* q_scale, const float* w, const uint8_t* k8,
                     const float* k_scale, float* scores, int64_t ld, uint32_t* hist) {
  if (hist)
    hipLaunchKernelGGL((index_score_kernel<RG, NPF, NT, true>), grid, dim3(kThreads), 0, s, b, q8,
                       q_scale, w, k8, k_scale, scores, ld, hist);
  else
    hipLaunchKernelGGL((index_score_kernel<RG, NPF, NT, false>), grid, dim3(kThreads), 0, s, b,
                       q8, q_scale, w, k8, k_scale, scores, ld, hist);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_score(const BatchArgs& b, const uint8_t* q8, const float* q_scale,
                              const float* w, const uint8_t* k8, const float* k_scale,
                              float* scores, int64_t ld, uint32_t* hist, hipStream_t s) {
  if (b.B == 0 || b.T == 0 || b.max_seqlen_k == 0) return hipSuccess;
  const int rg = b.max_q <= 1 ? 1 : (b.max_q <= 2 ? 2 : 4);
  const int groups = (b.max_q + rg - 1) / rg;
  const int total_pages = (b.max_seqlen_k + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE;
  const int chunks = (total_pages + kChunk - 1) / kChunk;
  dim3 grid(groups, chunks, b.B);
  if (rg == 1)
    return launch_rg<1, 8, true>(grid, s, b, q8, q_scale, w, k8, k_scale, scores, ld, hist);
  if (rg == 2)
    return launch_rg<2, 4, true>(grid, s, b, q8, q_scale, w, k8, k_scale, scores, ld, hist);
  if (groups == 1)
    return launch_rg<4, 2, true>(grid, s, b, q8, q_scale, w, k8, k_scale, scores, ld, hist);
  return launch_rg<4, 2, false>(grid, s, b, q8, q_scale, w, k8, k_scale, scores, ld, hist);
}

}  // namespace dsa
