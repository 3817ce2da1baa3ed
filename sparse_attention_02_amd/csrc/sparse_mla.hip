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
// heads, so each gathered latent row is read from HBM once per row.  Per
// tile of 32 selected tokens:
//   gather   slots come from a per-split table built once (position -> page
//            -> slot); each 1152-byte row goes straight from HBM into LDS
//            (buffer loads to LDS through a descriptor over the row, a
//            1024-byte and a 128-byte piece; row pitch 1184 bytes) into a
//            ring of three buffers.  Buffer loads, not global_load_lds: with
//            the latter in flight the compiler waits for every outstanding
//            LDS read (lgkmcnt(0)) wherever it needs one, which defeats the
//            operand read-ahead below;
//   S^T      = KV Q^T, wave w taking heads 16w .. 16w+15 (v_mfma_f32_16x16x32_bf16;
//            the latent part of its query is held in registers, the rope
//            part in LDS);
//   softmax  online, per head, in fp32 by the wave that owns the head; the
//            reference max is only raised when a score exceeds it by 2^8, so
//            the accumulator is rarely rescaled (the result does not depend
//            on the reference).  P goes to LDS in the MFMA operand layout,
//            with the rescale factor of each head;
//   O^T     += V^T P^T, wave w taking latent dims 64w .. 64w+63 for all 128
//            heads, so every value row is read from LDS once per tile rather
//            than once per head group.  V^T comes straight from the
//            token-major tile through transposing LDS reads
//            (ds_read_b64_tr_b16: four tokens of one dim per lane), in the
//            token order in which the S^T accumulator holds P.
// With several splits per row each writes its normalised partial output in
// fp16, scaled per (head, 64-dim slice) by a power of two, plus the slice
// scales and its lse, and a merge kernel combines them.  The output (or
// partial) leaves through LDS as whole 128-byte rows of one head.
// The loop is software-pipelined: step i runs the value product of tile i
// and the scores of tile i+1 while tile i+2 streams in, with one barrier per
// step.  Operand reads run ahead of the products that use them (two k-steps
// in S^T, one head block in O^T), fixed with scheduling fences.
#include <cfloat>

#include "device_common.h"

namespace dsa {
namespace {

constexpr int kThreads = 512;
// Row pitches are chosen for gfx950's LDS (64 banks of 4 bytes): a
// ds_read_b128 whose lanes l%16 pick rows and l/16 pick 16-byte columns is
// conflict-free when the pitch is 32 mod 64 bytes (measured: 1152 or 1168
// bytes cost 1.65-3x more).
constexpr int kKsPitch = 1184;                 // bytes per token row of the gathered tile
constexpr int kKsBytes = kMlaTile * kKsPitch;  // 37888
constexpr int kMaxChunk = 2048;                // selected tokens per split
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleMargin = 8.f;          // log2 units
constexpr int kQkAhead = 2;                    // S^T k-steps whose operands are in flight

constexpr int kDimsPerWave = DSA_MLA_DV / (kThreads / 64);  // 64

union Frag {
  uint4 u;
  v8bf v;
};

typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) void lds_void;

// V^T operand of a 16-dim block: lane (l16, g) receives dim d0 + l16 of
// tokens 4g .. 4g+3 and 16+4g .. 16+4g+3, i.e. k = 8g .. 8g+7 in the order
// the S^T accumulator hands out P.  For the 16 lanes of group g, lane L
// addresses token row 4g + L/4 (and 16 rows below) at dims d0 + 4(L%4).
__device__ __forceinline__ v8bf v_frag(const unsigned char* K, int d0, int l16, int g) {
  const unsigned char* p = K + (4 * g + (l16 >> 2)) * kKsPitch + (d0 + 4 * (l16 & 3)) * 2;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 16 * kKsPitch));
  const v8s x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(v8bf, x);
}

__device__ __forceinline__ v8bf lds_frag(const unsigned char* p) {
  Frag f;
  f.u = *reinterpret_cast<const uint4*>(p);
  return f.v;
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; a field at its maximum does not wait)
constexpr unsigned kWaitVmAll = 0x0f70;   // vmcnt(0)
constexpr unsigned kWaitLgkmAll = 0xc07f; // lgkmcnt(0)

// Waits for every global load this wave issued, including those that write
// LDS directly.  A builtin rather than inline assembly, so that the compiler
// knows those writes are complete.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(kWaitVmAll); }

// Work-group barrier over LDS only: each wave's LDS accesses complete before
// it arrives, but loads still streaming into another buffer keep going
// (__syncthreads' fence would wait for them too).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkmAll);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-stage LDS of the tile ring: the gathered tile, the P^T fragments of
// all 128 heads ([head block][lane]), each head's rescale factor and one
// flag per wave (some head of the wave was rescaled).  Three stages are
// separate variables so that the compiler can tell them apart.
struct Stage {
  unsigned char* K;
  uint4* P;
  float* alpha;
  uint8_t* raised;
};

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// two floats as fp16 (round to nearest even) in one word, the first low
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const h2v v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(h2v, w)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(h2v, w)[1];
}

// power of two s with m * s in [2^14, 2^15) for a finite m > 0 (1 otherwise,
// and clamped to the normal range): fp16 values of magnitude up to m keep 11
// significant bits and stay far from the fp16 maximum
__device__ __forceinline__ float half_scale(float m) {
  if (!(m > 0.f) || !(m < INFINITY)) return 1.f;
  const int e = (int)((__float_as_uint(m) >> 23) & 255u) - 127;  // floor(log2 m) for normal m
  const int k = min(127, max(-126, 14 - e));
  return __uint_as_float((uint32_t)(k + 127) << 23);
}

template <bool SPLIT>
__global__ __launch_bounds__(kThreads)
void sparse_mla_kernel(BatchArgs b, const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
                       const int32_t* __restrict__ idx, int k, float scale_log2,
                       uint16_t* __restrict__ out, float* __restrict__ lse,
                       uint16_t* __restrict__ opart, float* __restrict__ spart,
                       float* __restrict__ lpart, int n_split, int chunk,
                       int n_work, int per_xcd, int idx_mode) {
  __shared__ __attribute__((aligned(16))) unsigned char Ks0[kKsBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Ks1[kKsBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Ks2[kKsBytes];
  // P^T, rescale factors and flags of two consecutive tiles (by tile parity)
  __shared__ __attribute__((aligned(16))) uint4 Pl[2][8 * 64];
  __shared__ float al[2][DSA_MLA_HEADS];
  __shared__ __attribute__((aligned(8))) uint8_t rw[2][8];
  // rope part of the query (dims 512..575) as S^T operands: [k-step][wave][lane]
  __shared__ __attribute__((aligned(16))) uint4 Qr[2][8 * 64];
  __shared__ float fin_l[DSA_MLA_HEADS];    // 1 / softmax denominator of each head
  __shared__ int32_t slots[kMaxChunk];

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
  // entries past min(k, v) hold nothing in the dense form and in a compact
  // selection (the top-k writes its min(k, v) positions first, then -1):
  // their tiles, and splits made only of them, are skipped outright
  const int lim = idx_mode == kMlaDense || idx_mode == kMlaCompact ? min(k, v) : k;
  const int ntok = max(0, min(lim, j0 + chunk) - j0);
  const int ntiles = (ntok + kMlaTile - 1) / kMlaTile;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int head = wave * 16 + l16;

  // B operand of S^T: q[t, head, 32kk + 8g .. +8]; the latent part in
  // registers, the rope part (k-steps 16 and 17) in LDS
  v8bf qf[16];
  uint4 qr_pre[2];
  {
    const uint4* src =
        reinterpret_cast<const uint4*>(q + ((int64_t)t * DSA_MLA_HEADS + head) * DSA_MLA_DIM) + g;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      Frag f;
      f.u = src[4 * kk];
      qf[kk] = f.v;
    }
    qr_pre[0] = src[4 * 16];
    qr_pre[1] = src[4 * 17];
  }

  // position -> slot for the whole split (-1: skipped); paged entries are
  // slots already (only their range is checked); the dense form attends
  // every visible position, the entry being the position itself
  const int64_t n_slots = (int64_t)b.num_pages * DSA_PAGE_SIZE;
  for (int i = tid; i < ntiles * kMlaTile; i += kThreads) {
    int slot = -1;
    if (i < ntok) {
      const int s = idx_mode == kMlaDense ? j0 + i : idx[(int64_t)t * k + j0 + i];
      if (idx_mode == kMlaPaged) {
        device_check(b, s < -1 || s >= n_slots, DSA_CHECK_INDEX);
        if (s >= 0 && s < n_slots) slot = s;
      } else if (s >= 0 && s < v) {
        const int64_t sl = slot_of(b, bi, s);
        device_check(b, sl < 0, DSA_CHECK_PAGE_ID);
        if (sl >= 0) slot = (int)sl;
      } else {
        device_check(b, s != -1, DSA_CHECK_INDEX);
      }
    }
    slots[i] = slot;
  }
  // the query loads and the slot table's loads overlapped; all have landed
  // before the first gather is issued
  wait_vm_all();
  Qr[0][wave * 64 + lane] = qr_pre[0];
  Qr[1][wave * 64 + lane] = qr_pre[1];
  __syncthreads();

  // slots of a tile, one per lane: lane L holds token L % 32 (-1: skipped or
  // past the split)
  auto slot_vec = [&](int tile) -> int {
    return tile < ntiles ? slots[tile * kMlaTile + (lane & 31)] : -1;
  };
  // bit x: token x of the tile has a row
  auto tile_bits = [&](int sv) -> uint32_t { return (uint32_t)__ballot(sv >= 0); };

  // one tile, one token row at a time: wave w fetches rows 4w .. 4w+3, each
  // with a 1024-byte load (16 bytes a lane) and a 128-byte one (4 bytes on
  // each of 32 lanes; LDS-bound loads narrower than a dword still fill a
  // dword per lane) into the row's place in the tile.  A row's slot is the
  // same for the whole wave, so its address is a scalar base plus a fixed
  // lane offset (no per-lane address arithmetic); a skipped row re-reads a
  // valid one, so every row the products touch holds finite cache data.
  const uint32_t tail_ofs = 1024u + 4u * (uint32_t)lane;  // bytes 1024 .. 1151 of a row (lanes < 32)
  auto issue_gather = [&](int sv, uint32_t bits, unsigned char* dst) {
    if (bits == 0) return;
    const int fb = __builtin_amdgcn_readlane(sv, __builtin_ctz(bits));
#pragma unroll
    for (int i = 0; i < kMlaTile / 8; ++i) {
      const int r = 4 * wave + i;
      int slot = __builtin_amdgcn_readlane(sv, r);
      if (slot < 0) slot = fb;
      const uint16_t* row = kv + (int64_t)slot * DSA_MLA_DIM;
      unsigned char* d = dst + r * kKsPitch;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(row), (short)0, DSA_MLA_DIM * 2, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)d, 16, 16 * lane, 0, 0, 0);
      if (lane < 32)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(d + 1024), 4, tail_ofs, 0, 0, 0);
    }
  };

  // acc[db][hb][r] = O^T[dim 64w + 16db + 4g + r][head 16hb + l16]
  v4f acc[4][8];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) acc[db][hb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_ref = -FLT_MAX;  // reference max of this lane's head (log2 units)
  float l_run = 0.f;
  const int d_base = kDimsPerWave * wave;

  // S^T of a tile and its online softmax; P^T and the rescale factors go to
  // the tile's stage.  Straight-line code, so that the value product of the
  // previous tile can be scheduled into it.
  auto qk_softmax = [&](uint32_t mask, const Stage& st) {
    // S^T (32 tokens x 16 heads) = KV (32 x 576) . Q^T (576 x 16)
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    // the operands of k-step kk + kQkAhead are read while kk's products run;
    // the scheduling fences keep the compiler from regrouping them
    const unsigned char* kr = st.K + l16 * kKsPitch + g * 16;
    v8bf a0[kQkAhead + 1], a1[kQkAhead + 1];
#pragma unroll
    for (int d = 0; d < kQkAhead; ++d) {
      a0[d] = lds_frag(kr + 64 * d);
      a1[d] = lds_frag(kr + 16 * kKsPitch + 64 * d);
    }
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) {
      if (kk + kQkAhead < 18) {
        a0[(kk + kQkAhead) % (kQkAhead + 1)] = lds_frag(kr + 64 * (kk + kQkAhead));
        a1[(kk + kQkAhead) % (kQkAhead + 1)] = lds_frag(kr + 16 * kKsPitch + 64 * (kk + kQkAhead));
      }
      Frag qb;
      if (kk < 16) qb.v = qf[kk < 16 ? kk : 0];  // (the index guard only silences the unrolled tail)
      else qb.u = Qr[kk - 16][wave * 64 + lane];
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[kk % (kQkAhead + 1)], qb.v, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[kk % (kQkAhead + 1)], qb.v, s1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane holds tokens 4g + r (s0) and 16 + 4g + r (s1) of head `head`
    float z[8];
    if (mask == ~0u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[r] = s0[r] * scale_log2;
        z[4 + r] = s1[r] * scale_log2;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[r] = (mask >> (4 * g + r)) & 1u ? s0[r] * scale_log2 : -INFINITY;
        z[4 + r] = (mask >> (16 + 4 * g + r)) & 1u ? s1[r] * scale_log2 : -INFINITY;
      }
    }
    float tmax = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])),
                       fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
    {  // max over the four 16-lane rows (lanes l, l^16, l^32, l^48), in VALU
      const v2u x = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                                     false, false);
      tmax = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
      const v2u y = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                                     false, false);
      tmax = fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
    }
    // the reference starts at -FLT_MAX, below every finite score, so the
    // first finite maximum always raises it (with a factor of 0 for the
    // empty accumulator) and z - m_ref is never inf - inf
    const bool raise = tmax > m_ref + kRescaleMargin;
    const float m_new = raise ? tmax : m_ref;
    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
    l_run *= alpha;
    m_ref = m_new;
    st.alpha[head] = alpha;  // the four lanes of a head store the same value
    st.raised[wave] = __ballot(alpha != 1.f) != 0;
    float p[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) p[r] = __builtin_amdgcn_exp2f(z[r] - m_ref);
    const float psum = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    l_run += psum;
    st.P[wave * 64 + lane] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                        pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
  };

  // O^T (64 dims x 128 heads) += V^T (64 x 32) . P^T (32 x 128) for a tile
  // whose P^T is in its stage
  auto pv = [&](const Stage& st) {
    v8bf va[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) va[db] = v_frag(st.K, d_base + 16 * db, l16, g);
    // P^T of head block hb + 1 is read while hb's products run
    Frag pb[2];
    pb[0].u = st.P[lane];
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) {
      if (hb + 1 < 8) pb[(hb + 1) & 1].u = st.P[(hb + 1) * 64 + lane];
#pragma unroll
      for (int db = 0; db < 4; ++db)
        acc[db][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[db], pb[hb & 1].v, acc[db][hb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Step `tile`: the value product of `tile` and the scores of `tile + 1`,
  // while `tile + 2` streams into the third stage.  Carried between steps:
  // the token masks of `tile` and `tile + 1`, the slot vector of `tile + 2`.
  uint32_t bits_c = 0, bits_n1 = 0, bits_n2 = 0;
  int sv_n2 = -1;
  auto step = [&](int tile, const Stage& cur, const Stage& nx1, const Stage& nx2) {
    wait_vm_all();  // this wave's share of tile + 1 has landed
    lds_barrier();  // every share has; P^T of `tile` is complete; the third stage is free
    issue_gather(sv_n2, bits_n2, nx2.K);
    const int sv_n3 = slot_vec(tile + 3);
    const uint64_t rescaled = *reinterpret_cast<const uint64_t*>(cur.raised);
    if (bits_n1) qk_softmax(bits_n1, nx1);
    if (bits_c) {
      if (rescaled) {
#pragma unroll
        for (int hb = 0; hb < 8; ++hb) {
          const float a = cur.alpha[16 * hb + l16];
#pragma unroll
          for (int db = 0; db < 4; ++db) acc[db][hb] *= a;
        }
      }
      pv(cur);
    }
    bits_c = bits_n1;
    bits_n1 = bits_n2;
    bits_n2 = tile_bits(sv_n3);
    sv_n2 = sv_n3;
  };

  // stages of tiles 3i, 3i+1, 3i+2; P^T and the rescale data alternate by
  // tile parity
  auto stage = [&](unsigned char* K, int tile) {
    const int par = tile & 1;
    return Stage{K, Pl[par], al[par], rw[par]};
  };
  {
    const int sv0 = slot_vec(0), sv1 = slot_vec(1);
    sv_n2 = slot_vec(2);
    bits_c = tile_bits(sv0);
    bits_n1 = tile_bits(sv1);
    bits_n2 = tile_bits(sv_n2);
    issue_gather(sv0, bits_c, Ks0);
    wait_vm_all();
    lds_barrier();
    issue_gather(sv1, bits_n1, Ks1);
    if (bits_c) qk_softmax(bits_c, stage(Ks0, 0));
  }
  for (int tile = 0; tile < ntiles; tile += 3) {
    step(tile, stage(Ks0, tile), stage(Ks1, tile + 1), stage(Ks2, tile + 2));
    step(tile + 1, stage(Ks1, tile + 1), stage(Ks2, tile + 2), stage(Ks0, tile + 3));
    step(tile + 2, stage(Ks2, tile + 2), stage(Ks0, tile + 3), stage(Ks1, tile + 4));
  }

  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  const float lse_v = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  if (g == 0) fin_l[head] = l_tot > 0.f ? 1.f / l_tot : 0.f;
  lds_barrier();
  // lane holds O^T[d_base + 16db + 4g + r][16hb + l16].  The wave's 64
  // dims of each head leave as one 128-byte row: four head blocks at a time
  // are packed into an 8 KB LDS region of the wave (the ring is free now;
  // 16-byte chunks XOR-swizzled by row), then read back 16 bytes a lane
  // (eight lanes per row) and stored row by row.
  unsigned char* stage_out = (wave < 4 ? Ks0 : Ks1) + (wave & 3) * 8192;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int hq = 0; hq < 4; ++hq) {
      const int hb = 4 * pass + hq;
      const int h = 16 * hb + l16;
      const float inv = fin_l[h];
      float f = inv;
      if (SPLIT) {
        // the split's partial in fp16, scaled per (head, this wave's 64 dims)
        // by a power of two that puts its largest magnitude in [2^14, 2^15):
        // 11 significant bits, against 8 for the bf16 output
        float mx = 0.f;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(acc[db][hb][r]));
        {  // max over the four 16-lane rows, which hold the head's other dims
          const v2u x = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
          mx = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
          const v2u y = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
          mx = fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
        }
        const float sc = half_scale(mx * inv);
        f = inv * sc;
        if (g == 0)
          spart[(((int64_t)t * n_split + split) * (kThreads / 64) + wave) * DSA_MLA_HEADS + h] =
              1.f / sc;
      }
      const int row = 16 * hq + l16;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const v4f x = acc[db][hb];
        const int c = (2 * db + (g >> 1)) ^ (row & 7);
        *reinterpret_cast<uint2*>(stage_out + row * 128 + c * 16 + 8 * (g & 1)) =
            SPLIT ? make_uint2(pack_f16x2(x[0] * f, x[1] * f), pack_f16x2(x[2] * f, x[3] * f))
                  : make_uint2(pack_bf16x2(x[0] * f, x[1] * f), pack_bf16x2(x[2] * f, x[3] * f));
      }
    }
    uint16_t* dst = SPLIT ? opart + ((int64_t)t * n_split + split) * DSA_MLA_HEADS * DSA_MLA_DV
                          : out + (int64_t)t * DSA_MLA_HEADS * DSA_MLA_DV;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * i + (lane >> 3);
      const int cc = lane & 7;
      const uint4 w = *reinterpret_cast<const uint4*>(stage_out + row * 128 + ((cc ^ (row & 7)) * 16));
      *reinterpret_cast<uint4*>(dst + (int64_t)(64 * pass + row) * DSA_MLA_DV + d_base + 8 * cc) = w;
    }
  }
  if (g == 0) {
    if (!SPLIT) {
      if (lse) lse[(int64_t)t * DSA_MLA_HEADS + head] = lse_v;
    } else {
      lpart[((int64_t)t * n_split + split) * DSA_MLA_HEADS + head] = lse_v;
    }
  }
}

// out(t,h) = sum_j e^{lse_j - lse*} O_j / sum_j e^{lse_j - lse*},
// lse(t,h) = lse* + ln sum_j e^{lse_j - lse*}, lse* = max_j lse_j.
// One wave per (row, head), eight per work-group; lane l holds dims
// 8l .. 8l+7 (16-byte loads of the fp16 partials, one 16-byte bf16 store).
constexpr int kMergeWaves = 8;

// MANY: more than four splits, read in batches of eight (a separate
// instance, so that the common form keeps its smaller register footprint)
template <bool MANY>
__global__ __launch_bounds__(64 * kMergeWaves) void mla_merge_kernel(
    const uint16_t* __restrict__ opart, const float* __restrict__ spart,
    const float* __restrict__ lpart, int n_split, int64_t n_th, uint16_t* __restrict__ out,
    float* __restrict__ lse, int per_xcd) {
  // work-groups are dealt to the 8 XCDs round-robin; XCD x takes the x-th
  // eighth of the (row, head) range, the rows whose splits the attention ran
  // on that XCD, so the partials are read from the L2 that they were written to
  const int64_t wg = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  const int64_t th = wg * kMergeWaves + (threadIdx.x >> 6);  // t * 128 + h
  if (th >= n_th) return;
  const int64_t t = th / DSA_MLA_HEADS;
  const int h = (int)(th - t * DSA_MLA_HEADS);
  const int l = threadIdx.x & 63;
  const float* lp = lpart + t * n_split * DSA_MLA_HEADS + h;
  auto lse_of = [&](int j) { return lp[j * DSA_MLA_HEADS]; };
  // the power-of-two scale of this lane's 64-dim slice (written by wave l / 8)
  auto scale_of = [&](int j) {
    return spart[((t * n_split + j) * (kThreads / 64) + l / 8) * DSA_MLA_HEADS + h];
  };
  auto part_of = [&](int j) {
    return *reinterpret_cast<const uint4*>(
        opart + ((t * n_split + j) * DSA_MLA_HEADS + h) * DSA_MLA_DV + 8 * l);
  };
  uint16_t* o = out + th * DSA_MLA_DV + 8 * l;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f, mx = -INFINITY;
  // split j's share, in ascending j (the order fixes the rounding)
  auto add = [&](float lj, float u, uint4 hx) {
    const float wj = __expf(lj - mx);
    if (wj == 0.f) return;
    wsum += wj;
    const uint32_t wd[4] = {hx.x, hx.y, hx.z, hx.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[2 * q] += wj * (f16_lo(wd[q]) * u);
      a[2 * q + 1] += wj * (f16_hi(wd[q]) * u);
    }
  };
  if (!MANY) {
    // every load issued before any is used
    float lj[4], u[4];
    uint4 hx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int jj = min(j, n_split - 1);
      lj[j] = lse_of(jj);
      u[j] = scale_of(jj);
      hx[j] = part_of(jj);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < n_split) mx = fmaxf(mx, lj[j]);
    if (mx != -INFINITY) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < n_split) add(lj[j], u[j], hx[j]);
    }
  } else {
    // batches of 8 splits, each batch's loads issued before any is used
    // (one round trip per batch, not per split)
    constexpr int kB = 8;
    for (int j0 = 0; j0 < n_split; j0 += kB) {
      float lj[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) lj[u] = lse_of(min(j0 + u, n_split - 1));
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (j0 + u < n_split) mx = fmaxf(mx, lj[u]);
    }
    if (mx != -INFINITY) {
      for (int j0 = 0; j0 < n_split; j0 += kB) {
        float lj[kB], u_[kB];
        uint4 hx[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          const int jj = min(j0 + u, n_split - 1);
          lj[u] = lse_of(jj);
          u_[u] = scale_of(jj);
          hx[u] = part_of(jj);
        }
#pragma unroll
        for (int u = 0; u < kB; ++u)
          if (j0 + u < n_split) add(lj[u], u_[u], hx[u]);
      }
    }
  }
  if (mx == -INFINITY) {
    *reinterpret_cast<uint4*>(o) = make_uint4(0u, 0u, 0u, 0u);
    if (lse && l == 0) lse[th] = -INFINITY;
    return;
  }
  const float inv = 1.f / wsum;
  *reinterpret_cast<uint4*>(o) =
      make_uint4(pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv),
                 pack_bf16x2(a[4] * inv, a[5] * inv), pack_bf16x2(a[6] * inv, a[7] * inv));
  if (lse && l == 0) lse[th] = mx + logf(wsum);
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

int default_splits(const BatchArgs& b, int k, int wgs) {
  // at most `wgs` work-groups over the batch (256 = one per CU: a work-group
  // holds 156 KB of LDS, so a 257th waits for a whole second round -- 96 rows
  // in 3 splits took 131 us, in 2 splits 96 us), and at least 4 tiles per split: a
  // split's fixed costs (its slot table, the query load, its partial write
  // and its share of the merge) outweigh a tile's work below that (a single
  // row at k = 2048 runs its attention in 37 us with 16 splits, 60 us with 64)
  const int max_by_k = std::max(1, (k + 4 * kMlaTile - 1) / (4 * kMlaTile));
  if (b.T <= 0) return 1;
  int ns = wgs / b.T;
  ns = std::min(ns, std::min(max_by_k, kMaxSplits));
  return std::max(ns, 1);
}

MlaWs mla_ws_layout(const BatchArgs& b, int n_split) {
  MlaWs w{0, 0, 0, 0};
  if (n_split <= 1) return w;
  size_t off = 0;
  w.opart_off = off;  // fp16 partials [T][n_split][128][512]
  off = align_up(off + (size_t)b.T * n_split * DSA_MLA_HEADS * DSA_MLA_DV * 2, 256);
  w.spart_off = off;  // their scales [T][n_split][8 dim slices][128]
  off = align_up(off + (size_t)b.T * n_split * (kThreads / 64) * DSA_MLA_HEADS * 4, 256);
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
                             int n_split, void* ws, hipStream_t s, int idx_mode) {
  if (b.T == 0) return hipSuccess;
  int chunk, used;
  split_shape(k, n_split, &chunk, &used);
  const int n_work = b.T * used;
  const int per_xcd = (n_work + 7) / 8;
  const float scale_log2 = sm_scale * kLog2e;
  if (used == 1) {
    hipLaunchKernelGGL((sparse_mla_kernel<false>), dim3(8 * per_xcd), dim3(kThreads), 0, s, b, q,
                       kv, idx, k, scale_log2, out, lse, (uint16_t*)nullptr, (float*)nullptr,
                       (float*)nullptr, 1,
                       chunk, n_work, per_xcd, idx_mode);
    return hipGetLastError();
  }
  const MlaWs L = mla_ws_layout(b, used);
  char* base = static_cast<char*>(ws);
  uint16_t* opart = reinterpret_cast<uint16_t*>(base + L.opart_off);
  float* spart = reinterpret_cast<float*>(base + L.spart_off);
  float* lpart = reinterpret_cast<float*>(base + L.lpart_off);
  hipLaunchKernelGGL((sparse_mla_kernel<true>), dim3(8 * per_xcd), dim3(kThreads), 0, s, b, q, kv,
                     idx, k, scale_log2, out, lse, opart, spart, lpart, used, chunk, n_work, per_xcd,
                     idx_mode);
  const int64_t n_th = (int64_t)b.T * DSA_MLA_HEADS;
  const int64_t n_mwg = (n_th + kMergeWaves - 1) / kMergeWaves;
  const int m_per_xcd = (int)((n_mwg + 7) / 8);
  if (used <= 4)
    hipLaunchKernelGGL(mla_merge_kernel<false>, dim3((unsigned)(8 * m_per_xcd)),
                       dim3(64 * kMergeWaves), 0, s, opart, spart, lpart, used, n_th, out, lse,
                       m_per_xcd);
  else
    hipLaunchKernelGGL(mla_merge_kernel<true>, dim3((unsigned)(8 * m_per_xcd)),
                       dim3(64 * kMergeWaves), 0, s, opart, spart, lpart, used, n_th, out, lse,
                       m_per_xcd);
  return hipGetLastError();
}

}  // namespace dsa
