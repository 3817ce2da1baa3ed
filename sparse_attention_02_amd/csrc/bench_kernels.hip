// Measurement kernels (include/dsa_bench.h): HBM read ceilings for the access
// patterns of the path's kernels.  They compute nothing of the method.
#include <hip/hip_runtime.h>

#include <string>

#include "dsa.h"
#include "dsa_bench.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kStreamWGs = 2048;
constexpr int kStreamThreads = 256;
constexpr int kPageBytes = DSA_PAGE_SIZE * DSA_IDX_DIM;
constexpr int kRangePages = 128;
constexpr int kRing = 16;  // 1 KB loads in flight per wave: two pages

thread_local std::string g_bench_err;

// lane l of each 64-lane load reads bytes 16 l .. 16 l + 15 of a 1 KB run;
// work-group g takes runs g, g + kStreamWGs, ... (four loads issued before use)
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const v4i* __restrict__ p,
                                                                      int64_t n16,
                                                                      uint32_t* __restrict__ sink) {
  const int64_t lanes = (int64_t)kStreamWGs * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  v4i acc = {0, 0, 0, 0};
  for (; i + 3 * lanes < n16; i += 4 * lanes) {
    const v4i a = __builtin_nontemporal_load(p + i);
    const v4i b = __builtin_nontemporal_load(p + i + lanes);
    const v4i c = __builtin_nontemporal_load(p + i + 2 * lanes);
    const v4i d = __builtin_nontemporal_load(p + i + 3 * lanes);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += lanes) acc ^= __builtin_nontemporal_load(p + i);
  const uint32_t f = (uint32_t)(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if (f == 0x9e3779b9u) *sink = f;  // practically never: keeps the loads
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// one work-group = one request x one 128-page range; wave w reads pages
// w, w + 4, ...; each page as eight contiguous 1 KB buffer loads, the ring
// holding two pages' loads
__global__ __launch_bounds__(256, 2) void key_stream_kernel(const uint8_t* __restrict__ k8,
                                                            int num_pages,
                                                            const int32_t* __restrict__ pages,
                                                            int max_pages, const int32_t* lens,
                                                            int max_seqlen_k,
                                                            uint32_t* __restrict__ sink) {
  const int bi = blockIdx.y;
  int L = lens[bi];
  L = L < 0 ? 0 : (L > max_seqlen_k ? max_seqlen_k : L);
  const int p_begin = blockIdx.x * kRangePages;
  const int p_end = min(p_begin + kRangePages, (L + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE);
  if (p_begin >= p_end) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int np = max(0, (p_end - p_begin - wave + 3) / 4);
  const int32_t* pt = pages + (int64_t)bi * max_pages;
  const int my = lane < np ? pt[p_begin + wave + 4 * lane] : -1;
  auto page_id = [&](int i) { return i < np ? __builtin_amdgcn_readlane(my, i) : -1; };
  auto rsrc = [&](int pg) {
    const bool ok = pg >= 0 && pg < num_pages;
    return page_rsrc(k8 + (int64_t)(ok ? pg : 0) * kPageBytes, ok ? kPageBytes : 0);
  };
  v4i ring[kRing];
#pragma unroll
  for (int q = 0; q < kRing; ++q)
    ring[q] = __builtin_amdgcn_raw_buffer_load_b128(rsrc(page_id(q / 8)), 16 * lane, 1024 * (q % 8), 2);
  v4i acc = {0, 0, 0, 0};
  for (int i0 = 0; i0 < np; i0 += 2) {
#pragma unroll
    for (int q = 0; q < kRing; ++q) {
      acc ^= ring[q];
      __builtin_amdgcn_sched_barrier(0);
      ring[q] = __builtin_amdgcn_raw_buffer_load_b128(rsrc(page_id(i0 + 2 + q / 8)), 16 * lane,
                                                      1024 * (q % 8), 2);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const uint32_t f = (uint32_t)(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if (f == 0x9e3779b9u) *sink = f;
}

int bench_fail(const char* msg) {
  g_bench_err = msg;
  return DSA_ERR_INVALID_ARG;
}

}  // namespace

extern "C" {

int dsa_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || (bytes & 15) || ((uintptr_t)src & 15))
    return bench_fail("src and sink must be set, src and bytes 16-byte multiples");
  if (bytes == 0) return DSA_OK;
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamWGs), dim3(kStreamThreads), 0,
                     (hipStream_t)stream, static_cast<const v4i*>(src), (int64_t)(bytes / 16),
                     sink);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

int dsa_bench_key_stream_read(const uint8_t* k8_cache, int32_t num_pages, const int32_t* page_table,
                              int32_t batch, int32_t max_pages_per_req, const int32_t* seqlens_k,
                              int32_t max_seqlen_k, uint32_t* sink, void* stream) {
  if (batch < 0 || num_pages < 0 || max_seqlen_k < 0 || max_pages_per_req < 0)
    return bench_fail("negative size");
  if ((int64_t)max_pages_per_req * DSA_PAGE_SIZE < max_seqlen_k)
    return bench_fail("max_pages_per_req * 64 < max_seqlen_k");
  if (batch == 0 || max_seqlen_k == 0) return DSA_OK;
  if (!k8_cache || !page_table || !seqlens_k || !sink || ((uintptr_t)k8_cache & 15))
    return bench_fail("NULL or misaligned pointer");
  const int pages = (max_seqlen_k + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE;
  const dim3 grid((pages + kRangePages - 1) / kRangePages, batch);
  hipLaunchKernelGGL(key_stream_kernel, grid, dim3(256), 0, (hipStream_t)stream, k8_cache,
                     num_pages, page_table, max_pages_per_req, seqlens_k, max_seqlen_k, sink);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

}  // extern "C"
