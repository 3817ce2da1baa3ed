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
// One work-group (8 waves, two per SIMD) owns one (row, split) and all 128
// heads, so each gathered latent row is read from HBM once per row.  Wave w
// owns heads 16w .. 16w+15: its query fragment (16 heads x 576) and its
// output accumulator (512 dims x 16 heads, fp32) stay in registers
// (v_mfma_f32_16x16x32_bf16).  Per tile of 32 selected tokens:
//   gather   slots come from a per-split table built once (position -> page
//            -> slot); the 1152-byte rows go straight from HBM into LDS with
//            global_load_lds_dwordx4 (row pitch 1168 bytes), double-buffered:
//            tile i+1 streams in while tile i computes;
//   transpose the first 512 dims into a [dim][token] copy so that the value
//            product has its contraction (token) dim contiguous;
//   S^T      = KV Q^T (32 tokens x 16 heads per wave);
//   softmax  online, per head, in fp32; the reference max is only raised
//            when a score exceeds it by 2^8, so the accumulator is rarely
//            rescaled (the result does not depend on the reference);
//   O^T     += V^T P^T (512 dims x 16 heads), P taken straight from the S^T
//            accumulator layout (the token order of the transposed copy is
//            permuted to match it).
#include "device_common.h"

namespace dsa {
namespace {

constexpr int kThreads = 512;
// Row pitches are chosen for gfx950's LDS (64 banks of 4 bytes): a
// ds_read_b128 whose lanes l%16 pick rows and l/16 pick 16-byte columns is
// conflict-free when the pitch is 32 mod 64 bytes (measured: 1152 or 1168
// bytes cost 1.65-3x more).
constexpr int kKsPitch = 1184;                 // bytes per token row of the gathered tile
constexpr int kKsChunks = kKsPitch / 16;       // 74 (72 data + 2 pad)
constexpr int kKsLoads = (kMlaTile * kKsChunks + 63) / 64;  // 37 wave-wide 1 KB loads
constexpr int kKsBytes = kKsLoads * 1024;      // 37888
constexpr int kVtPitch = 96;                   // bytes per latent-dim row of the transposed tile
constexpr int kMaxChunk = 2048;                // selected tokens per split
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleMargin = 8.f;          // log2 units

union Frag {
  uint4 u;
  v8bf v;
};

__device__ __forceinline__ v8bf lds_frag(const unsigned char* p) {
  Frag f;
  f.u = *reinterpret_cast<const uint4*>(p);
  return f.v;
}

// column of token 4q+r in a row of the transposed tile: the order in which the
// S^T accumulator (16x16 layout: lane group g holds tokens 4g..4g+3 and
// 16+4g..16+4g+3) hands P to the value product
__device__ __forceinline__ int quad_pos(int q) { return 8 * (q & 3) + 4 * (q >> 2); }

template <bool SPLIT>
__global__ __launch_bounds__(kThreads)
void sparse_mla_kernel(BatchArgs b, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                       const int32_t* __restrict__ idx, int k, float scale_log2,
                       uint16_t* __restrict__ out, float* __restrict__ lse,
                       float* __restrict__ opart, float* __restrict__ lpart, int n_split, int chunk,
                       int n_work, int per_xcd) {
  __shared__ __attribute__((aligned(16))) unsigned char Ks[2][kKsBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Vt[DSA_MLA_DV * kVtPitch];
  __shared__ int32_t slots[kMaxChunk];
  __shared__ int32_t tile_fb[kMaxChunk / kMlaTile];    // a valid slot of the tile, -1 if none
  __shared__ uint32_t tile_mask[kMaxChunk / kMlaTile];  // bit x: token x of the tile is valid

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
  const int ntok = max(0, min(k, j0 + chunk) - j0);
  const int ntiles = (ntok + kMlaTile - 1) / kMlaTile;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int head = wave * 16 + l16;

  // position -> slot for the whole split (-1: skipped)
  for (int i = tid; i < ntiles * kMlaTile; i += kThreads) {
    int slot = -1;
    if (i < ntok) {
      const int s = idx[(int64_t)t * k + j0 + i];
      if (s >= 0 && s < v) {
        const int64_t sl = slot_of(b, bi, s);
        if (sl >= 0) slot = (int)sl;
      }
    }
    slots[i] = slot;
  }
  __syncthreads();
  for (int tt = tid; tt < ntiles; tt += kThreads) {
    int fb = -1;
    uint32_t mask = 0;
    for (int x = 0; x < kMlaTile; ++x) {
      const int sl = slots[tt * kMlaTile + x];
      if (sl >= 0) {
        mask |= 1u << x;
        if (fb < 0) fb = sl;
      }
    }
    tile_fb[tt] = fb;
    tile_mask[tt] = mask;
  }
  __syncthreads();

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

  // one tile: 37 wave-wide loads of 64 x 16 bytes; lane L of load n fills
  // byte 16*(64n + L) of the buffer = token (64n+L)/73, chunk (64n+L)%73
  auto issue_gather = [&](int tile, int buf) {
    const int fb = tile_fb[tile];
    if (fb < 0) return;
    for (int n = wave; n < kKsLoads; n += kThreads / 64) {
      const int c = 64 * n + lane;
      const int tok = c / kKsChunks;
      int cc = c - tok * kKsChunks;
      int slot = tok < kMlaTile ? slots[tile * kMlaTile + tok] : -1;
      if (slot < 0) slot = fb;  // padding lanes and skipped tokens re-read a valid row
      if (cc >= 72) cc = 0;  // pad chunks
      const uint16_t* src = kv + (int64_t)slot * DSA_MLA_DIM + cc * 8;
      __builtin_amdgcn_global_load_lds(src, Ks[buf] + n * 1024, 16, 0, 0);
    }
  };

  v4f acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference max of this lane's head (log2 units)
  float l_run = 0.f;

  if (ntiles > 0) issue_gather(0, 0);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile in Ks[buf]; every wave is done with the previous tile
    if (tile + 1 < ntiles) issue_gather(tile + 1, buf ^ 1);
    const bool live = tile_fb[tile] >= 0;
    if (live) {
      // transpose dims 0..511: lane (qd = lane/8, dc = 8*wave + lane%8) reads
      // 4 token rows of one 16-byte column (lanes 0-7 read 128 contiguous
      // bytes of a row, lanes 8-15 the row 4 below: disjoint banks) and
      // writes its 8 dims in a lane-rotated order so that the 8 rows written
      // together by lanes 0-7 fall in different banks
      const unsigned char* K = Ks[buf];
      {
        const int rot = lane & 7;
        const int qd = lane >> 3;
        const int dc = 8 * wave + rot;
        const uint4 r0 = *reinterpret_cast<const uint4*>(K + (4 * qd + 0) * kKsPitch + dc * 16);
        const uint4 r1 = *reinterpret_cast<const uint4*>(K + (4 * qd + 1) * kKsPitch + dc * 16);
        const uint4 r2 = *reinterpret_cast<const uint4*>(K + (4 * qd + 2) * kKsPitch + dc * 16);
        const uint4 r3 = *reinterpret_cast<const uint4*>(K + (4 * qd + 3) * kKsPitch + dc * 16);
        const uint32_t w0[4] = {r0.x, r0.y, r0.z, r0.w};
        const uint32_t w1[4] = {r1.x, r1.y, r1.z, r1.w};
        const uint32_t w2[4] = {r2.x, r2.y, r2.z, r2.w};
        const uint32_t w3[4] = {r3.x, r3.y, r3.z, r3.w};
        const int pos = quad_pos(qd);
        // dims (2wi, 2wi+1) of the 4 tokens: low and high halves of word wi
        uint32_t lo_e[4], hi_e[4], lo_o[4], hi_o[4];
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          lo_e[wi] = (w0[wi] & 0xffffu) | (w1[wi] << 16);
          hi_e[wi] = (w2[wi] & 0xffffu) | (w3[wi] << 16);
          lo_o[wi] = (w0[wi] >> 16) | (w1[wi] & 0xffff0000u);
          hi_o[wi] = (w2[wi] >> 16) | (w3[wi] & 0xffff0000u);
        }
#pragma unroll
        for (int step = 0; step < 8; ++step) {
          const int e = (step + rot) & 7;  // this lane's dim at this step
          const int wi = e >> 1;
          uint32_t lo = lo_e[0], hi = hi_e[0];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (wi == c) {
              lo = (e & 1) ? lo_o[c] : lo_e[c];
              hi = (e & 1) ? hi_o[c] : hi_e[c];
            }
          }
          *reinterpret_cast<uint2*>(Vt + (8 * dc + e) * kVtPitch + pos * 2) = make_uint2(lo, hi);
        }
      }
    }
    __syncthreads();
    if (!live) continue;

    // S^T (32 tokens x 16 heads) = KV (32 x 576) . Q^T (576 x 16)
    const unsigned char* K = Ks[buf];
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
      const v8bf a0 = lds_frag(K + l16 * kKsPitch + (4 * kk + g) * 16);
      const v8bf a1 = lds_frag(K + (16 + l16) * kKsPitch + (4 * kk + g) * 16);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[kk], s1, 0, 0, 0);
    }
    // lane holds tokens 4g + r (s0) and 16 + 4g + r (s1) of head `head`
    const uint32_t mask = tile_mask[tile];
    float z[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = s0[r] * scale_log2;
      z[4 + r] = s1[r] * scale_log2;
    }
    if (mask != 0xffffffffu) {  // a tile with skipped tokens (rare)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!((mask >> (4 * g + r)) & 1u)) z[r] = -INFINITY;
        if (!((mask >> (16 + 4 * g + r)) & 1u)) z[4 + r] = -INFINITY;
      }
    }
    float tmax = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])),
                       fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const bool raise = tmax > m_ref + kRescaleMargin || (m_ref == -INFINITY && tmax > -INFINITY);
    if (__ballot(raise)) {
      const float m_new = raise ? tmax : m_ref;
      const float alpha = m_ref == -INFINITY ? 0.f : exp2f(m_ref - m_new);
      if (__ballot(alpha != 1.f && m_ref != -INFINITY)) {
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] *= alpha;
      }
      l_run *= alpha;
      m_ref = m_new;
    }
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      p[r] = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[r] - m_ref);
      psum += p[r];
    }
    l_run += psum;
    Frag pf;
    pf.u = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7]));
    // O^T (512 x 16) += V^T (512 x 32) . P^T (32 x 16)
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      const v8bf a = lds_frag(Vt + (16 * mt + l16) * kVtPitch + 16 * g);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf.v, acc[mt], 0, 0, 0);
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_v = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  // lane holds O^T[16mt + 4g + r][head]
  if (!SPLIT) {
    uint16_t* o = out + ((int64_t)t * DSA_MLA_HEADS + head) * DSA_MLA_DV + 4 * g;
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      const v4f x = acc[mt];
      *reinterpret_cast<uint2*>(o + 16 * mt) =
          make_uint2(pack_bf16x2(x[0] * inv, x[1] * inv), pack_bf16x2(x[2] * inv, x[3] * inv));
    }
    if (lse && g == 0) lse[(int64_t)t * DSA_MLA_HEADS + head] = lse_v;
  } else {
    float* o = opart + (((int64_t)t * n_split + split) * DSA_MLA_HEADS + head) * DSA_MLA_DV + 4 * g;
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      const v4f x = acc[mt];
      *reinterpret_cast<float4*>(o + 16 * mt) =
          make_float4(x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv);
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

// tokens per split (a multiple of the tile, at most kMaxChunk) and the
// splits actually used
void split_shape(int k, int n_split, int* chunk, int* used) {
  int c = (k + n_split - 1) / n_split;
  c = (c + kMlaTile - 1) / kMlaTile * kMlaTile;
  c = std::min(c, kMaxChunk);
  *chunk = c;
  *used = (k + c - 1) / c;
}

}  // namespace

int default_splits(const BatchArgs& b, int k) {
  const int max_by_k = std::max(1, (k + kMlaTile - 1) / kMlaTile);
  if (b.T <= 0) return 1;
  int ns = (256 + b.T - 1) / b.T;
  ns = std::min(ns, std::min(max_by_k, kMaxSplits));
  return std::max(ns, 1);
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

int mla_splits_used(int k, int n_split) {
  int chunk, used;
  split_shape(k, n_split, &chunk, &used);
  return used;
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

}  // namespace dsa
