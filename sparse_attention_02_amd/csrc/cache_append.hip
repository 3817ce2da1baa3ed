// Cache append for gfx950: the new tokens of a decode (or prefill) step go
// into the two paged caches the sparse decode reads.
//
// Per new token (query row t of request b, cached at position
// p = L_b - n_b + j, slot = page_table[b][p / 64] * 64 + p % 64):
//   indexer cache  its 128-dim key is quantised to OCP e4m3fn with one fp32
//                  scale = max_d |k_d| / 448 (1 for an all-zero key): code_d =
//                  e4m3(k_d / scale), rounded to nearest even;
//   latent cache   its 576-wide bf16 row (512 latent + 64 rope) is stored as is.
// ("MTP and sparse attention: NSA and DSA", new demands on inference engines:
// the indexer keys are a second paged cache beside the latent, 128 FP8 bytes
// plus a 4-byte scale per token; "[SGLang] NSA", forward_decode: the new
// tokens' latent rows are written to the paged pool before the attention.)
//
// One wave per token: lane l holds key dims 2l and 2l+1, the amax is a wave
// reduction, and the hardware conversion v_cvt_pk_fp8_f32 (round to nearest
// even) packs the two codes; the 1152-byte latent row moves as 72 16-byte
// chunks.  The kernel is bound by the latency of one dependent chain per
// token (a few microseconds at decode sizes) and by HBM beyond that.
#include "device_common.h"

namespace dsa {
namespace {

constexpr int kAppendWaves = 4;  // tokens per work-group
constexpr int kKvChunks = DSA_MLA_DIM * 2 / 16;  // 72 chunks of 16 bytes

__global__ __launch_bounds__(64 * kAppendWaves) void cache_append_kernel(
    BatchArgs b, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ kv_new,
    uint8_t* __restrict__ k8, float* __restrict__ ks, uint16_t* __restrict__ kv) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kAppendWaves + (threadIdx.x >> 6);
  if (t >= b.T) return;
  const int bi = row_request(b.cu, b.B, t);
  const int n = b.cu[bi + 1] - b.cu[bi];
  const int pos = clamp_len(b, b.lens[bi]) - n + (t - b.cu[bi]);
  // a request whose cached length does not hold its rows
  device_check(b, pos < 0, DSA_CHECK_METADATA);
  if (pos < 0) return;
  const int64_t slot = slot_of(b, bi, pos);
  device_check(b, slot < 0, DSA_CHECK_PAGE_ID);
  if (slot < 0) return;  // page id outside the pool: nothing is written

  const uint32_t kb = reinterpret_cast<const uint32_t*>(k_new + (int64_t)t * DSA_IDX_DIM)[lane];
  const float x0 = __uint_as_float(kb << 16);
  const float x1 = __uint_as_float(kb & 0xffff0000u);
  float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  // |k_d / scale| <= 448 up to one rounding, inside e4m3fn's finite range
  const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(x0 / scale, x1 / scale, 0, false);
  reinterpret_cast<uint16_t*>(k8 + slot * DSA_IDX_DIM)[lane] = (uint16_t)(packed & 0xffff);
  if (lane == 0) ks[slot] = scale;

  const uint4* src = reinterpret_cast<const uint4*>(kv_new + (int64_t)t * DSA_MLA_DIM);
  uint4* dst = reinterpret_cast<uint4*>(kv + slot * DSA_MLA_DIM);
  dst[lane] = src[lane];
  if (lane < kKvChunks - 64) dst[64 + lane] = src[64 + lane];
}

}  // namespace

hipError_t launch_cache_append(const BatchArgs& b, const uint16_t* k_new, const uint16_t* kv_new,
                               uint8_t* k8, float* ks, uint16_t* kv, hipStream_t s) {
  if (b.T == 0) return hipSuccess;
  hipLaunchKernelGGL(cache_append_kernel, dim3((unsigned)((b.T + kAppendWaves - 1) / kAppendWaves)),
                     dim3(64 * kAppendWaves), 0, s, b, k_new, kv_new, k8, ks, kv);
  return hipGetLastError();
}

}  // namespace dsa
