// Device helpers shared by the HIP kernels of the DSA path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Records `flag` in the device check word when `bad` holds (builds with
// DSA_DEVICE_CHECKS; compiled out otherwise).  A vector atomic OR.
__device__ __forceinline__ void device_check(const BatchArgs& b, bool bad, uint32_t flag) {
#ifdef DSA_DEVICE_CHECKS
  if (bad && b.check) atomicOr(b.check, flag);
#else
  (void)b;
  (void)bad;
  (void)flag;
#endif
}

// Request owning query row t: the largest b with cu[b] <= t (rows of a
// request with no rows are skipped because cu[b] == cu[b+1]).
__device__ __forceinline__ int row_request(const int32_t* cu, int B, int t) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Tokens a request may address, from the host scalars: the cache length is
// clamped to the page-table width and to max_seqlen_k so that bad device
// metadata never leads outside the described buffers.
__device__ __forceinline__ int clamp_len(const BatchArgs& b, int L) {
  int cap = b.max_seqlen_k;
  int pcap = b.max_pages * DSA_PAGE_SIZE;
  if (pcap < cap) cap = pcap;
  device_check(b, L < 0 || L > cap, DSA_CHECK_METADATA);
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// Row j of request bi (n rows, L cached tokens) sees L - n + 1 + j tokens.
__device__ __forceinline__ int row_visible(const BatchArgs& b, int bi, int t) {
  int c0 = b.cu[bi];
  int n = b.cu[bi + 1] - c0;
  device_check(b, n > b.max_q, DSA_CHECK_METADATA);
  int L = clamp_len(b, b.lens[bi]);
  int v = L - n + 1 + (t - c0);
  return v < 0 ? 0 : (v > L ? L : v);
}

// Physical slot of logical position s of request bi, or -1 when the page id
// is outside the pool.
__device__ __forceinline__ int64_t slot_of(const BatchArgs& b, int bi, int s) {
  int page = b.pages[(int64_t)bi * b.max_pages + (s >> 6)];
  if (page < 0 || page >= b.num_pages) return -1;
  return (int64_t)page * DSA_PAGE_SIZE + (s & 63);
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// two floats to bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace dsa
