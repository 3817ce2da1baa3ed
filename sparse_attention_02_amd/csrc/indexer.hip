// Lightning-indexer scan for gfx950.
//
// I(t,s) = q_scale(t) * k_scale(s) * sum_h w(t,h) * max(0, q8(t,h) . k8(s))
// ("MTP and sparse attention: NSA and DSA", DSA bullet; the per-token scales
// are positive, so they factor out of the ReLU exactly).
//
// One work-group = one request x one group of RG query rows x one chunk of
// KC cache pages.  Each of its 4 waves owns 16 of the 64 tokens of a
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
#include <algorithm>

#include "device_common.h"

namespace dsa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// pages per work-group of the row-group form: 128 where the grid still
// holds several work-groups per CU (a prefill chunk: the queries and
// weights are loaded once per 128 pages instead of per 16, 2.59 -> 1.96 ms
// for 4096 rows on 65536 tokens), else 16
constexpr int kChunkSmall = 16;
constexpr int kChunkLarge = 128;
constexpr int kChunkLargeMinWGs = 2048;
#ifndef DSA_SCAN_TARGET_WGS
#define DSA_SCAN_TARGET_WGS 1024
#endif
#ifndef DSA_SCAN_SHARED_TARGET_WGS
#define DSA_SCAN_SHARED_TARGET_WGS 2048
#endif
// 1 KB key loads in flight per wave of the page form (one or two rows):
// two pages (16) took 202.6 us on the 128K batch, 20 took 207.1, 24 took 204.8
#ifndef DSA_SCAN_QN1
#define DSA_SCAN_QN1 16
#endif
#ifndef DSA_SCAN_QN2
#define DSA_SCAN_QN2 16
#endif
constexpr int kScanTargetWGs = DSA_SCAN_TARGET_WGS;
constexpr int kScanQN1 = DSA_SCAN_QN1;
constexpr int kScanQN2 = DSA_SCAN_QN2;
#ifndef DSA_SCAN_STAGE_PAGES
#define DSA_SCAN_STAGE_PAGES 128
#endif
constexpr int kStagePages = DSA_SCAN_STAGE_PAGES;  // most pages per work-group
// beside another kernel (the attention of multi-layer-indexer mode) the scan
// uses work-groups of at most 64 pages and half the LDS: finer-grained
// work-groups free CUs for the other kernel sooner (two streams over the
// 48-request ragged batch: 0.266 ms with 64-page work-groups, 0.289 ms with
// 128, against 0.31 ms on one stream)
constexpr int kSharedStagePages = 64;
constexpr int kSharedTargetWGs = DSA_SCAN_SHARED_TARGET_WGS;

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
template <int RG, int NPF, bool NT, bool HIST, int KC>
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
  const int p_begin = chunk * KC;
  const int p_end = min(p_begin + KC, (vmax + 63) >> 6);
  if (p_begin >= p_end) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15;  // key within the wave's 16
  const int g = lane >> 4;  // k-group of the operands / row of the result

  if (HIST) {
    for (int i = threadIdx.x; i < RG * kTopkBins; i += kThreads) lh[i] = 0u;
  }

  // page i of the chunk (past the end: the last page again; bad ids read
  // page 0 and score -inf).  The chunk's page ids are staged in LDS once, so
  // a page's address costs an in-order LDS read rather than a scalar load
  // (whose wait, scalar loads returning out of order, is always a full one).
  const int32_t* ptab = b.pages + (int64_t)bi * b.max_pages;
  const int lane_key = 16 * wave + j;
  __shared__ int lpid[KC];
  for (int i = threadIdx.x; i < KC; i += kThreads) lpid[i] = ptab[min(p_begin + i, p_end - 1)];
  __syncthreads();
  auto page_id = [&](int i) { return lpid[min(i, KC - 1)]; };
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
  // (the staging barrier above also ordered the histogram's zeroing)

  int pg_next = page_id(NPF);  // the page whose keys are loaded next
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const v8i kcur = kf[i % NPF];
    const float kscur = ksr[i % NPF];
    if (i + NPF < KC) {
      const int pg = pg_next;
      pg_next = page_id(i + NPF + 1);
      kf[i % NPF] = NT ? load_frag_nt(key_ptr(pg)) : load_frag(key_ptr(pg));
      ksr[i % NPF] = *scale_ptr(pg);
    }
    // the products of (row, head tile) x = 4 r + m, one ahead of the ReLU * w
    // that reads them: two accumulators in turn, so each MFMA runs while the
    // previous one's results are consumed (with one accumulator the next
    // product waits for the reads, and the results for the product)
    float sum[RG];
    v4f acc_cur =
        __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[0][0], kcur, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int x = 0; x < 4 * RG; ++x) {
      const int r = x >> 2, m = x & 3;
      v4f acc_next = zero;
      if (x + 1 < 4 * RG)
        acc_next = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[(x + 1) >> 2][(x + 1) & 3],
                                                                   kcur, zero, 0, 0, 0, 0, 0, 0);
      if (m == 0) sum[r] = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[r] = fmaf(wr[r][m][e], relu(acc_cur[e]), sum[r]);
      acc_cur = acc_next;
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
    if (p_begin + i < p_end && g < nr && s < vis_g) {
      // a page whose id is outside the pool holds no keys: -inf
      const bool ok = page_ok(page_id(i));
      device_check(b, !ok, DSA_CHECK_PAGE_ID);
      const float sc = ok ? mine * qs_g * kscur : -INFINITY;
      device_check(b, sc != sc, DSA_CHECK_NAN_SCORE);
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

template <int RG, int NPF, bool NT, int KC>
hipError_t launch_rg(dim3 grid, hipStream_t s, const BatchArgs& b, const uint8_t* q8,
                     const float* q_scale, const float* w, const uint8_t* k8,
                     const float* k_scale, float* scores, int64_t ld, uint32_t* hist) {
  if (hist)
    hipLaunchKernelGGL((index_score_kernel<RG, NPF, NT, true, KC>), grid, dim3(kThreads), 0, s, b,
                       q8, q_scale, w, k8, k_scale, scores, ld, hist);
  else
    hipLaunchKernelGGL((index_score_kernel<RG, NPF, NT, false, KC>), grid, dim3(kThreads), 0, s,
                       b, q8, q_scale, w, k8, k_scale, scores, ld, hist);
  return hipGetLastError();
}

// ---- decode form: one wave per page ------------------------------------
//
// For requests of at most two query rows (a decode token, plus one MTP
// draft) each key page is scanned by one wave on its own.  The page's 64
// keys are the four 16-key column tiles of the MFMA, so after the ReLU * w
// reduction over heads the 64 lanes hold the page's 64 scores in order and
// each row's scores leave in one 256-byte store.  The cross-lane part of the
// head reduction is a reduce-scatter over the four 16-lane rows with the
// permlane32 / permlane16 swaps, with no LDS.  Keys arrive through buffer
// loads whose descriptor spans exactly one page: a page past the wave's range
// or with an id outside the pool gets a zero-size descriptor, so its loads
// return zeros without touching memory.
//
// Each key load is contiguous: lane l reads bytes 16 l .. 16 l + 15 of a
// 1 KB run (eight whole keys), so a 16-lane quarter of the wave touches two
// 128-byte lines.  Loading the MFMA operand layout directly (lane (j, g)
// reading 16 bytes of key j) touches sixteen lines per quarter and held a
// load-only copy of the scan at 192 us on the 128K batch against 162 us for
// contiguous loads.  A wave turns each 2 KB column tile into the operand
// layout through its own 2 KB of LDS (one write and one read of 16 bytes
// per lane and half-tile); the buffer is XOR-swizzled so that the writes
// have no bank conflicts.
constexpr int kPageWaves = 4;
constexpr int kPageKeyBytes = DSA_PAGE_SIZE * DSA_IDX_DIM;
constexpr int kTileBytes = 16 * DSA_IDX_DIM;  // one column tile: 16 keys
constexpr int kBufNT = 2;  // nontemporal cache policy of a buffer load

typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// lane (j, g) holds p[c] for column tile c, summed over its own heads; the
// result in lane (j, g) is the sum over all four g of column tile g
__device__ __forceinline__ float reduce_scatter4(const float p[4]) {
  const v2u a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]),
                                                 false, false);
  const v2u c = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]),
                                                 false, false);
  const float x = __uint_as_float(a[0]) + __uint_as_float(a[1]);  // tile 0 | tile 2
  const float y = __uint_as_float(c[0]) + __uint_as_float(c[1]);  // tile 1 | tile 3
  const v2u d = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false,
                                                 false);
  return __uint_as_float(d[0]) + __uint_as_float(d[1]);
}

template <int RG, int QN, bool HIST, int STAGE>
__global__ __launch_bounds__(kThreads, 2) void index_score_page_kernel(
    BatchArgs b, const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const float* __restrict__ w, const uint8_t* __restrict__ k8,
    const float* __restrict__ k_scale, float* __restrict__ scores, int64_t ld,
    uint32_t* __restrict__ hist, int chunk_pages) {
  // first-digit histogram of each row, two 16-bit counts per word (a
  // work-group scores at most STAGE * 64 <= 8192 positions of a row, so no
  // count reaches 2^16)
  static_assert(STAGE * DSA_PAGE_SIZE < 65536, "16-bit histogram counts");
  __shared__ uint32_t lh[HIST ? RG * kTopkBins / 2 : 1];
  // the work-group's scores, written out in one burst at the end
  __shared__ float lsc[RG][STAGE * DSA_PAGE_SIZE];
  // each wave's column tile in transit from the load layout to the operand
  // layout
  __shared__ __attribute__((aligned(16))) uint8_t ltr[kPageWaves][kTileBytes];
  const int chunk = blockIdx.x;
  const int bi = blockIdx.y;
  const int c0 = b.cu[bi];
  const int n = b.cu[bi + 1] - c0;  // 0 .. RG rows (the launch checks max_q <= RG)
  device_check(b, n < 0 || n > RG, DSA_CHECK_METADATA);
  if (n <= 0 || n > RG) return;
  const int L = clamp_len(b, b.lens[bi]);
  const int p_begin = chunk * chunk_pages;
  const int p_end = min(p_begin + chunk_pages, (L + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE);
  if (p_begin >= p_end) return;

  const int lane = threadIdx.x & 63;
  // wave-uniform (readfirstlane tells the compiler so: the page descriptors
  // built from it then stay in scalar registers)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15;
  const int g = lane >> 4;
  if (HIST) {
    for (int i = threadIdx.x; i < RG * kTopkBins / 2; i += kThreads) lh[i] = 0u;
  }

  // the wave's pages are p_begin + wave + 4i, i < np (np <= 64: one id per lane)
  const int np = max(0, (p_end - p_begin - wave + kPageWaves - 1) / kPageWaves);
  const int32_t* ptab = b.pages + (int64_t)bi * b.max_pages;
  const int my_pid = lane < np ? ptab[p_begin + wave + kPageWaves * lane] : -1;
  auto page_id = [&](int i) { return i < np ? __builtin_amdgcn_readlane(my_pid, i) : -1; };
  auto page_ok = [&](int pg) { return pg >= 0 && pg < b.num_pages; };

  // A operands and weights of each row (rows past the request's last repeat it)
  v8i qf[RG][4];
  float wr[RG][4][4];
  float qs[RG];
  int vis[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int t = c0 + min(r, n - 1);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      qf[r][m] = load_frag(q8 + ((int64_t)t * DSA_IDX_HEADS + 16 * m + j) * DSA_IDX_DIM + 32 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) wr[r][m][e] = w[(int64_t)t * DSA_IDX_HEADS + 16 * m + 4 * g + e];
    }
    qs[r] = q_scale[t];
    vis[r] = r < n ? min(L, max(0, L - n + 1 + r)) : 0;
  }

  // key ring: QN 1 KB loads in flight per wave.  Load x of a page holds keys
  // 8x .. 8x+7 (lane l: key 8x + l/8, bytes 16 (l % 8) .. 16 (l % 8) + 15).
  // Chunk q of the wave's stream (page q / 8, load q % 8) lives in register
  // set q % QN; as soon as a pair of chunks has been handed to the tile
  // transposition, its registers take chunks q + QN and q + QN + 1, so no
  // register of the ring is copied.  The page loop is unrolled over GP pages
  // (one full turn of the ring), which makes every register index static.
  static_assert(QN % 2 == 0 && QN >= 8 && QN <= 32, "ring of 8 .. 32 chunks");
  constexpr int GP = (QN % 8 == 0 ? QN : (QN % 4 == 0 ? 2 * QN : 4 * QN)) / 8;
  v4i kr[QN];
  float ksr[GP];
  auto key_rsrc = [&](int pg) {
    const bool ok = page_ok(pg);
    return page_rsrc(k8 + (int64_t)(ok ? pg : 0) * kPageKeyBytes, ok ? kPageKeyBytes : 0);
  };
  const int voff = 16 * lane;
  auto load_part = [&](__amdgpu_buffer_rsrc_t rs, int x) {
    // the 1 KB offset rides in the scalar offset, so all loads share one
    // address register
    return __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 1024 * x, kBufNT);
  };
  auto load_scale = [&](int pg) {
    const bool ok = page_ok(pg);
    const __amdgpu_buffer_rsrc_t sr = page_rsrc(
        k_scale + (int64_t)(ok ? pg : 0) * DSA_PAGE_SIZE, ok ? DSA_PAGE_SIZE * 4 : 0);
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sr, 4 * lane, 0, kBufNT));
  };
  // transposition: key kk's 16-byte chunk ch sits at kk * 128 + 16 * (ch ^
  // 2 ((kk / 2) % 4)).  The swizzle leaves the pairs (2p, 2p + 1) in order
  // and ignores key bit 3, so the second half-tile's write and the second
  // operand read are immediate offsets of the first (1024 and 16 bytes).
  // Writes are free of bank conflicts; the operand reads conflict two-way.
  uint8_t* tw = ltr[wave];
  const int w_ofs = (lane >> 3) * DSA_IDX_DIM + (((lane & 7) ^ (2 * ((lane >> 4) & 3))) << 4);
  const int r_ofs = j * DSA_IDX_DIM + (((2 * g) ^ (2 * ((j >> 1) & 3))) << 4);
  auto transpose = [&](v4i lo_half, v4i hi_half) {
    *reinterpret_cast<v4i*>(tw + w_ofs) = lo_half;
    *reinterpret_cast<v4i*>(tw + w_ofs + 8 * DSA_IDX_DIM) = hi_half;
    const v4i a = *reinterpret_cast<const v4i*>(tw + r_ofs);
    const v4i c = *reinterpret_cast<const v4i*>(tw + r_ofs + 16);
    return v8i{a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
  };
#pragma unroll
  for (int q = 0; q < QN; ++q) kr[q] = load_part(key_rsrc(page_id(q / 8)), q % 8);
  ksr[0] = load_scale(page_id(0));
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  for (int i0 = 0; i0 < np; i0 += GP) {
#pragma unroll
    for (int u = 0; u < GP; ++u) {
      const int i = i0 + u;
      const int pg = page_id(i);
      // every wave runs whole groups of GP pages; past np the pages are
      // zero-size (their loads read nothing) and nothing is stored
      float part[RG][4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // the tile's operand through LDS; its two ring registers then take
        // the chunks QN ahead (the fences keep the loads after the LDS
        // writes that read those registers, and the MFMAs after the loads,
        // so the loads are in flight as early as possible)
        const int q = 8 * u + 2 * c;  // chunk within the group (a multiple of QN starts it)
        const v8i kb = transpose(kr[q % QN], kr[(q + 1) % QN]);
        __builtin_amdgcn_sched_barrier(0);
        {
          const int qn = q + QN;
          const __amdgpu_buffer_rsrc_t nr = key_rsrc(page_id(i0 + qn / 8));
          kr[q % QN] = load_part(nr, qn % 8);
          kr[(q + 1) % QN] = load_part(nr, (qn + 1) % 8);
        }
        __builtin_amdgcn_sched_barrier(0);
        v4f acc[RG][4];
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
          for (int m = 0; m < 4; ++m)
            acc[r][m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[r][m], kb, zero, 0,
                                                                      0, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          float sum = 0.f;
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) sum = fmaf(wr[r][m][e], relu(acc[r][m][e]), sum);
          // the empty asm pins the reduction here: left alone, the optimiser
          // sinks it to the end of the page, which keeps the MFMA results of
          // all four tiles live at once
          asm volatile("" : "+v"(sum));
          part[r][c] = sum;
        }
        // one tile's MFMA results live at a time (the other waves of the
        // SIMD overlap their MFMAs with this epilogue)
        __builtin_amdgcn_sched_barrier(0);
      }
      const int lp = wave + kPageWaves * i;  // page within the work-group's range
      const int pos = (p_begin + lp) * DSA_PAGE_SIZE + lane;
      // a page whose id is outside the pool holds no keys: its positions
      // score -inf, below every real score
      const bool ok = page_ok(pg);
      device_check(b, i < np && !ok, DSA_CHECK_PAGE_ID);
      const float ks = ksr[u];
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const float tot = reduce_scatter4(part[r]);
        if (i < np && r < n && pos < vis[r]) {
          const float sc = ok ? tot * qs[r] * ks : -INFINITY;
          device_check(b, sc != sc, DSA_CHECK_NAN_SCORE);
          lsc[r][lp * DSA_PAGE_SIZE + lane] = sc;
          if (HIST) {
            const uint32_t key = float_key(sc);
            atomicAdd(&lh[r * (kTopkBins / 2) + (key >> 22)], 1u << (((key >> 21) & 1u) * 16));
          }
        }
      }
      // the next page's key scales, one page ahead of their use
      ksr[(u + 1) % GP] = load_scale(page_id(i + 1));
    }
  }

  __syncthreads();
  // scores of the range, row by row: positions below the row's visible
  // count, in 16-byte stores where the row is aligned.  The stores are
  // nontemporal: written while the key stream is being read, cached writes
  // cost the scan far more than their share of the bytes.
  const int base = p_begin * DSA_PAGE_SIZE;
  const int span = (p_end - p_begin) * DSA_PAGE_SIZE;
  for (int r = 0; r < n; ++r) {
    const int lim = min(span, vis[r] - base);
    float* row = scores + (int64_t)(c0 + r) * ld + base;
    const bool vec = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
    for (int x = 4 * threadIdx.x; x < lim; x += 4 * kThreads) {
      if (vec && x + 4 <= lim) {
        __builtin_nontemporal_store(*reinterpret_cast<const v4f*>(&lsc[r][x]),
                                    reinterpret_cast<v4f*>(row + x));
      } else {
        for (int e = 0; e < 4 && x + e < lim; ++e) __builtin_nontemporal_store(lsc[r][x + e], row + x + e);
      }
    }
  }
  if (HIST) {
    for (int i = threadIdx.x; i < n * (kTopkBins / 2); i += kThreads) {
      const uint32_t c = lh[i];
      if (c) {
        uint32_t* gh = hist + (int64_t)(c0 + i / (kTopkBins / 2)) * kTopkBins + 2 * (i % (kTopkBins / 2));
        if (c & 0xffffu) atomicAdd(gh, c & 0xffffu);
        if (c >> 16) atomicAdd(gh + 1, c >> 16);
      }
    }
  }
}

template <int RG, int QN, int STAGE>
hipError_t launch_page(int chunk_pages, int chunks, hipStream_t s, const BatchArgs& b,
                       const uint8_t* q8, const float* q_scale, const float* w, const uint8_t* k8,
                       const float* k_scale, float* scores, int64_t ld, uint32_t* hist) {
  const dim3 grid(chunks, b.B);
  if (hist)
    hipLaunchKernelGGL((index_score_page_kernel<RG, QN, true, STAGE>), grid, dim3(kThreads), 0,
                       s, b, q8, q_scale, w, k8, k_scale, scores, ld, hist, chunk_pages);
  else
    hipLaunchKernelGGL((index_score_page_kernel<RG, QN, false, STAGE>), grid, dim3(kThreads), 0,
                       s, b, q8, q_scale, w, k8, k_scale, scores, ld, hist, chunk_pages);
  return hipGetLastError();
}

template <int RG, int QN>
hipError_t launch_page_sized(bool shared, int total_pages, hipStream_t s, const BatchArgs& b,
                             const uint8_t* q8, const float* q_scale, const float* w,
                             const uint8_t* k8, const float* k_scale, float* scores, int64_t ld,
                             uint32_t* hist) {
  // pages per work-group: about the target number of work-groups over the
  // batch (sized for its longest request), at most STAGE pages (<= 64 per wave)
  const int stage = shared ? kSharedStagePages : kStagePages;
  const int target = shared ? kSharedTargetWGs : kScanTargetWGs;
  const int64_t all = (int64_t)total_pages * b.B;
  int cp = (int)std::min<int64_t>(stage, (all + target - 1) / target);
  cp = std::max(kPageWaves, (cp + kPageWaves - 1) / kPageWaves * kPageWaves);
  const int chunks = (total_pages + cp - 1) / cp;
  if (shared)
    return launch_page<RG, QN, kSharedStagePages>(cp, chunks, s, b, q8, q_scale, w, k8, k_scale,
                                                   scores, ld, hist);
  return launch_page<RG, QN, kStagePages>(cp, chunks, s, b, q8, q_scale, w, k8, k_scale, scores,
                                           ld, hist);
}

}  // namespace

hipError_t launch_index_score(const BatchArgs& b, const uint8_t* q8, const float* q_scale,
                              const float* w, const uint8_t* k8, const float* k_scale,
                              float* scores, int64_t ld, uint32_t* hist, hipStream_t s,
                              bool shared) {
  if (b.B == 0 || b.T == 0 || b.max_seqlen_k == 0) return hipSuccess;
  const int total_pages = (b.max_seqlen_k + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE;
  if (b.max_q <= 2) {
    if (b.max_q <= 1)
      return launch_page_sized<1, kScanQN1>(shared, total_pages, s, b, q8, q_scale, w, k8,
                                             k_scale, scores, ld, hist);
    return launch_page_sized<2, kScanQN2>(shared, total_pages, s, b, q8, q_scale, w, k8, k_scale,
                                           scores, ld, hist);
  }
  const int groups = (b.max_q + 3) / 4;
  const int64_t large = (int64_t)groups * ((total_pages + kChunkLarge - 1) / kChunkLarge) * b.B;
  if (large >= kChunkLargeMinWGs) {
    const dim3 grid(groups, (total_pages + kChunkLarge - 1) / kChunkLarge, b.B);
    if (groups == 1)
      return launch_rg<4, 2, true, kChunkLarge>(grid, s, b, q8, q_scale, w, k8, k_scale, scores,
                                                ld, hist);
    return launch_rg<4, 2, false, kChunkLarge>(grid, s, b, q8, q_scale, w, k8, k_scale, scores, ld,
                                               hist);
  }
  const dim3 grid(groups, (total_pages + kChunkSmall - 1) / kChunkSmall, b.B);
  if (groups == 1)
    return launch_rg<4, 2, true, kChunkSmall>(grid, s, b, q8, q_scale, w, k8, k_scale, scores, ld,
                                              hist);
  return launch_rg<4, 2, false, kChunkSmall>(grid, s, b, q8, q_scale, w, k8, k_scale, scores, ld,
                                             hist);
}

}  // namespace dsa
