// Sparse absorbed-MLA decode for gfx950: split-KV online softmax over the
// selected latent rows, then a log-sum-exp merge of the splits.
//
// Per query row t and head h, over the selected positions S_t:
//   z(s) = sm_scale * q(t,h) . kv(s)          (576 dims: 512 latent + 64 rope)
//   out(t,h) = sum_s softmax(z)(s) * kv(s)[0:512],  lse(t,h) = ln sum_s e^z(s)
// ("MTP and sparse attention: NSA and DSA", DSA bullet and per-pair cost;
// the split / merge structure is stages 2 and 3 of the sparse decode in
// "Deepseek Details", section DSA).
//
// One work-group (8 waves, 512 threads) owns one (row, split) and all 128
// heads, so each gathered latent row is read from HBM once per row.  Wave w
// owns heads 16w .. 16w+15; its query fragment stays in registers.  Per tile
// of 32 selected tokens:
//   gather   positions -> physical slots through the page table; 16-byte
//            loads of the 1152-byte rows into LDS (row pitch 1168 bytes);
//   transpose the first 512 dims into a [dim][token] copy in LDS so that the
//            value product has its contraction (token) dim contiguous;
//   S^T      = KV Q^T on v_mfma_f32_16x16x32_bf16 (tokens x heads);
//   softmax  online, per head, in fp32 (max over the tile by two xor steps);
//   O^T     += V^T P^T on the same MFMA (512 dims x 16 heads per wave), with
//            P taken straight from the S^T accumulator layout (the token
//            order of the transposed copy is permuted to match it).
#include "device_common.h"

namespace dsa {
namespace {

constexpr int kThreads = 512;
constexpr int kKsPitch = 1168;  // bytes per token row of the gathered tile
constexpr int kVtPitch = 80;    // bytes per latent-dim row of the transposed tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

union Frag {
  uint4 u;
  v8bf v;
};

__device__ __forceinline__ v8bf lds_frag(const unsigned char* p) {
  Frag f;
  f.u = *reinterpret_cast<const uint4*>(p);
  return f.v;
}

template <bool SPLIT>
__global__ __launch_bounds__(kThreads, 1) void sparse_mla_kernel(
    BatchArgs b, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ idx, int k, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, float* __restrict__ opart, float* __restrict__ lpart, int n_split,
    int chunk, int n_work, int per_xcd) {
  __shared__ __attribute__((aligned(16))) unsigned char Ks[kMlaTile * kKsPitch];
  __shared__ __attribute__((aligned(16))) unsigned char Vt[DSA_MLA_DV * kVtPitch];
  __shared__ int64_t rowoff[kMlaTile];

  // consecutive work items land on the same XCD (work-groups are dealt to
  // the 8 XCDs round-robin), so the splits and the MTP rows of a request
  // share that XCD's L2
  const int work = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (work >= n_work) return;
  const int t = work / n_split;
  const int split = work - t * n_split;
  const int bi = row_request(b.cu, b.B, t);
  const int v = row_visible(b, bi, t);
  const int j0 = split * chunk;
  const int j1 = min(k, j0 + chunk);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int head = wave * 16 + l16;

  // B operand of S^T: q[t, head, 32kk + 8g .. +8]
  v8bf qf[18];
  {
    const uint4* src =
        reinterpret_cast<const uint4*>(q + ((int64_t)t * DSA_MLA_HEADS + head) * DSA_MLA_DIM) + g;
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
      Frag f;
      f.u = src[4 * kk];
      qf[kk] = f.v;
    }
  }

  v4f acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  for (int j = j0; j < j1; j += kMlaTile) {
    if (tid < kMlaTile) {
      int64_t off = -1;
      if (j + tid < j1) {
        const int s = idx[(int64_t)t * k + j + tid];
        if (s >= 0 && s < v) {
          const int64_t slot = slot_of(b, bi, s);
          if (slot >= 0) off = slot * DSA_MLA_DIM;
        }
      }
      rowoff[tid] = off;
    }
    __syncthreads();

    // gather: 32 tokens x 72 chunks of 16 bytes, in two batches of loads
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint4 val[3];
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        const int c = tid + (3 * half + r) * kThreads;
        val[r] = make_uint4(0u, 0u, 0u, 0u);
        if (3 * half + r < 5 && c < kMlaTile * 72) {
          const int tok = c / 72, cc = c - tok * 72;
          const int64_t off = rowoff[tok];
          if (off >= 0) val[r] = *reinterpret_cast<const uint4*>(kv + off + cc * 8);
        }
      }
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        const int c = tid + (3 * half + r) * kThreads;
        if (3 * half + r < 5 && c < kMlaTile * 72) {
          const int tok = c / 72, cc = c - tok * 72;
          *reinterpret_cast<uint4*>(Ks + tok * kKsPitch + cc * 16) = val[r];
        }
      }
    }
    __syncthreads();

    // transpose dims 0..511: thread = (token quad qd, 8-dim chunk dc)
    {
      const int qd = tid & 7;
      const int dc = tid >> 3;
      const uint4 r0 = *reinterpret_cast<const uint4*>(Ks + (4 * qd + 0) * kKsPitch + dc * 16);
      const uint4 r1 = *reinterpret_cast<const uint4*>(Ks + (4 * qd + 1) * kKsPitch + dc * 16);
      const uint4 r2 = *reinterpret_cast<const uint4*>(Ks + (4 * qd + 2) * kKsPitch + dc * 16);
      const uint4 r3 = *reinterpret_cast<const uint4*>(Ks + (4 * qd + 3) * kKsPitch + dc * 16);
      const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w};
      const uint32_t w1[4] = {r1.x, r1.y, r1.z, r1.w};
      const uint32_t w2[4] = {r2.x, r2.y, r2.z, r2.w};
      const uint32_t w3[4] = {r3.x, r3.y, r3.z, r3.w};
      // token 4qd + r sits at column 8(qd & 3) + 4(qd >> 2) + r, the order in
      // which the S^T accumulator hands P to the value product
      const int pos = 8 * (qd & 3) + 4 * (qd >> 2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1;
        uint32_t lo, hi;
        if (e & 1) {
          lo = (w0[wi] >> 16) | (w1[wi] & 0xffff0000u);
          hi = (w2[wi] >> 16) | (w3[wi] & 0xffff0000u);
        } else {
          lo = (w0[wi] & 0xffffu) | (w1[wi] << 16);
          hi = (w2[wi] & 0xffffu) | (w3[wi] << 16);
        }
        *reinterpret_cast<uint2*>(Vt + (8 * dc + e) * kVtPitch + pos * 2) = make_uint2(lo, hi);
      }
    }
    __syncthreads();

    // S^T (32 tokens x 16 heads) = KV (32 x 576) . Q^T (576 x 16)
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
      const v8bf a0 = lds_frag(Ks + l16 * kKsPitch + (4 * kk + g) * 16);
      const v8bf a1 = lds_frag(Ks + (16 + l16) * kKsPitch + (4 * kk + g) * 16);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[kk], s1, 0, 0, 0);
    }
    // lane holds tokens 4g + r (s0) and 16 + 4g + r (s1) of head `head`
    float z[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = rowoff[4 * g + r] >= 0 ? s0[r] * scale_log2 : -INFINITY;
      z[4 + r] = rowoff[16 + 4 * g + r] >= 0 ? s1[r] * scale_log2 : -INFINITY;
    }
    float tmax = z[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) tmax = fmaxf(tmax, z[r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    float alpha = 1.f;
    float p[8];
    if (m_new == -INFINITY) {
#pragma unroll
      for (int r = 0; r < 8; ++r) p[r] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int r = 0; r < 8; ++r) p[r] = exp2f(z[r] - m_new);
    }
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) psum += p[r];
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] *= alpha;
    }
    Frag pf;
    pf.u = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7]));
    // O^T (512 x 16) += V^T (512 x 32) . P^T (32 x 16)
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      const v8bf a = lds_frag(Vt + (16 * mt + l16) * kVtPitch + 16 * g);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf.v, acc[mt], 0, 0, 0);
    }
    __syncthreads();
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  // lane holds O^T[16mt + 4g + r][head]
  if (!SPLIT) {
    uint16_t* o = out + ((int64_t)t * DSA_MLA_HEADS + head) * DSA_MLA_DV + 4 * g;
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      const v4f a = acc[mt];
      *reinterpret_cast<uint2*>(o + 16 * mt) =
          make_uint2(pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv));
    }
    if (lse && g == 0) lse[(int64_t)t * DSA_MLA_HEADS + head] = lse_v;
  } else {
    float* o = opart + (((int64_t)t * n_split + split) * DSA_MLA_HEADS + head) * DSA_MLA_DV + 4 * g;
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      const v4f a = acc[mt];
      *reinterpret_cast<float4*>(o + 16 * mt) = make_float4(a[0] * inv, a[1] * inv, a[2] * inv,
                                                            a[3] * inv);
    }
    if (g == 0) lpart[((int64_t)t * n_split + split) * DSA_MLA_HEADS + head] = lse_v;
  }
}

// out(t,h) = sum_j e^{lse_j - lse*} O_j / sum_j e^{lse_j - lse*},
// lse(t,h) = lse* + ln sum_j e^{lse_j - lse*}, lse* = max_j lse_j.
__global__ __launch_bounds__(128) void mla_merge_kernel(const float* __restrict__ opart,
                                                        const float* __restrict__ lpart,
                                                        int n_split, uint16_t* __restrict__ out,
                                                        float* __restrict__ lse) {
  const int64_t th = blockIdx.x;  // t * 128 + h
  const int64_t t = th / DSA_MLA_HEADS;
  const int h = (int)(th - t * DSA_MLA_HEADS);
  const float* lp = lpart + t * n_split * DSA_MLA_HEADS + h;
  float mx = -INFINITY;
  for (int j = 0; j < n_split; ++j) mx = fmaxf(mx, lp[j * DSA_MLA_HEADS]);
  uint16_t* o = out + th * DSA_MLA_DV + 4 * threadIdx.x;
  if (mx == -INFINITY) {
    *reinterpret_cast<uint2*>(o) = make_uint2(0u, 0u);
    if (lse && threadIdx.x == 0) lse[th] = -INFINITY;
    return;
  }
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  for (int j = 0; j < n_split; ++j) {
    const float wj = __expf(lp[j * DSA_MLA_HEADS] - mx);
    if (wj == 0.f) continue;
    wsum += wj;
    const float4 x = *reinterpret_cast<const float4*>(
        opart + ((t * n_split + j) * DSA_MLA_HEADS + h) * DSA_MLA_DV + 4 * threadIdx.x);
    a.x += wj * x.x;
    a.y += wj * x.y;
    a.z += wj * x.z;
    a.w += wj * x.w;
  }
  const float inv = 1.f / wsum;
  *reinterpret_cast<uint2*>(o) =
      make_uint2(pack_bf16x2(a.x * inv, a.y * inv), pack_bf16x2(a.z * inv, a.w * inv));
  if (lse && threadIdx.x == 0) lse[th] = mx + logf(wsum);
}

}  // namespace

int default_splits(const BatchArgs& b, int k) {
  const int max_by_k = std::max(1, (k + kMlaTile - 1) / kMlaTile);
  if (b.T <= 0) return 1;
  int ns = (256 + b.T - 1) / b.T;
  ns = std::min(ns, std::min(max_by_k, kMaxSplits));
  return std::max(ns, 1);
}

// tokens per split (a multiple of the tile) and the splits actually used
static void split_shape(int k, int n_split, int* chunk, int* used) {
  int c = (k + n_split - 1) / n_split;
  c = (c + kMlaTile - 1) / kMlaTile * kMlaTile;
  *chunk = c;
  *used = (k + c - 1) / c;
}

MlaWs mla_ws_layout(const BatchArgs& b, int n_split) {
  MlaWs w{0, 0, 0};
  if (n_split <= 1) return w;
  size_t off = 0;
  w.opart_off = off;
  off = align_up(off + (size_t)b.T * n_split * DSA_MLA_HEADS * DSA_MLA_DV * 4, 256);
  w.lpart_off = off;
  off = align_up(off + (size_t)b.T * n_split * DSA_MLA_HEADS * 4, 256);
  w.total = off;
  return w;
}

hipError_t launch_sparse_mla(const BatchArgs& b, const uint16_t* q, const uint16_t* kv,
                             const int32_t* idx, int k, float sm_scale, uint16_t* out, float* lse,
                             int n_split, void* ws, hipStream_t s) {
  if (b.T == 0) return hipSuccess;
  int chunk, used;
  split_shape(k, n_split, &chunk, &used);
  const int n_work = b.T * used;
  const int per_xcd = (n_work + 7) / 8;
  const float scale_log2 = sm_scale * kLog2e;
  if (used == 1) {
    hipLaunchKernelGGL((sparse_mla_kernel<false>), dim3(8 * per_xcd), dim3(kThreads), 0, s, b, q,
                       kv, idx, k, scale_log2, out, lse, (float*)nullptr, (float*)nullptr, 1,
                       chunk, n_work, per_xcd);
    return hipGetLastError();
  }
  const MlaWs L = mla_ws_layout(b, used);
  char* base = static_cast<char*>(ws);
  float* opart = reinterpret_cast<float*>(base + L.opart_off);
  float* lpart = reinterpret_cast<float*>(base + L.lpart_off);
  hipLaunchKernelGGL((sparse_mla_kernel<true>), dim3(8 * per_xcd), dim3(kThreads), 0, s, b, q, kv,
                     idx, k, scale_log2, out, lse, opart, lpart, used, chunk, n_work, per_xcd);
  hipLaunchKernelGGL(mla_merge_kernel, dim3((unsigned)(b.T * DSA_MLA_HEADS)), dim3(128), 0, s,
                     opart, lpart, used, out, lse);
  return hipGetLastError();
}

int mla_splits_used(int k, int n_split) {
  int chunk, used;
  split_shape(k, n_split, &chunk, &used);
  return used;
}

}  // namespace dsa
