// Masked multi-head attention in the expanded form, for prefills short
// enough that DSA's absorbed sparse attention costs more than attending
// densely.  Per row t and head h, over the positions s the row attends:
//   z(s) = sm_scale * (q_nope(t,h) . W_UK(h) c(s) + q_rope(t,h) . r(s))
//   out(t,h) = sum_s softmax(z)(s) W_UV(h) c(s)
// with c(s), r(s) the 512 latent and 64 rope dims of the cached row
// ("MTP and sparse attention: NSA and DSA": dense prefill runs this
// expanded form at 2*H*(128+64) + 2*H*128 FLOPs per pair against the
// absorbed form's 2*H*(512+64) + 2*H*512, and the V3.2 report emulates the
// sparse selection in it with a mask -- the caveat on short-sequence
// prefill).  Three kernels:
//   expand   K(h,s) = W_UK(h) c(s) and V(h,s) = W_UV(h) c(s) for every
//            cached position of each request (bf16, fp32 accumulation), and
//            the rope dims copied next to them;
//   mask     one bit per (row, position): the position is attended (listed
//            in the row's selection, or visible when there is no selection)
//            and on a page inside the pool;
//   attend   flash attention over 64-key tiles of K, rope and V staged in
//            LDS, 128 query rows of one head per work-group.
#include <algorithm>
#include <cfloat>
#include <type_traits>

#include "device_common.h"

namespace dsa {
namespace {

constexpr int kH = DSA_MLA_HEADS;  // 128 heads
constexpr int kDn = 128;           // up-projected dims per head (keys and values)
constexpr int kDr = 64;            // rope dims, shared by the heads
constexpr int kC = 512;            // latent dims
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

union Frag {
  uint4 u;
  v8bf v;
};

__device__ __forceinline__ v8bf as_frag(uint4 u) {
  Frag f;
  f.u = u;
  return f.v;
}

// ---------------------------------------------------------------- expand
//
// One work-group: head h of one request over a share of its positions, 8
// waves.  Waves 0-3 form K = W_UK(h) c, waves 4-7 V = W_UV(h) c, each for 32
// of the 128 dims, with its 32 rows of W held in registers for the whole
// run (the A operands of v_mfma_f32_16x16x32_bf16 for all 16 k-steps), so W
// is read once.  The latent rows stream through LDS in blocks of 64
// positions, double-buffered: one 1 KB DMA per row (its 512 latent dims, a
// buffer load to LDS through a descriptor over the row), chunk c of row r
// stored at chunk c ^ (r & 15) so that the B-operand reads (16 rows at one
// 16-byte column) are free of bank conflicts; a k-step's B operands are
// read while the previous k-step's products run (buffer loads rather than
// global_load_lds, with which in flight the compiler would wait for every
// outstanding LDS read, not only the k-step's).  Each lane
// ends with 4 consecutive dims of one position: one 8-byte store.  A
// block's slots and their validity come from its DMA issue (no page-table
// loads before the stores), and the rope dims of block j are copied by the
// work-groups of head j mod 128, so no head's work-groups carry all of it.
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kExpPos = 64;
constexpr int kExpThreads = 512;
constexpr int kExpRow = kC * 2;  // 1024 bytes of latent per row in LDS

__global__ __launch_bounds__(kExpThreads, 1) void mha_expand_kernel(
    BatchArgs b, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ w_uk,
    const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ kn, uint16_t* __restrict__ vn,
    uint16_t* __restrict__ rope, int lp, int n_share) {
  __shared__ __attribute__((aligned(16))) unsigned char lat[2][kExpPos * kExpRow];  // 128 KB
  const int h = blockIdx.x;
  const int share = blockIdx.y;
  const int bi = blockIdx.z;
  const int L = clamp_len(b, b.lens[bi]);
  const int nblk = (L + kExpPos - 1) / kExpPos;
  // blocks share, share + n_share, ... of the request
  if (share >= nblk) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int which = wave >> 2;    // 0: keys, 1: values
  const int d0 = 32 * (wave & 3);  // first of the wave's 32 dims

  // the wave's W rows as A operands: wf[db][kk] = W(h)[d0 + 16 db + l16][32 kk + 8 g .. +7]
  v8bf wf[2][16];
  {
    const uint16_t* W = (which ? w_uv : w_uk) + ((int64_t)h * kDn + d0 + l16) * kC + 8 * g;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int kk = 0; kk < 16; ++kk)
        wf[db][kk] = as_frag(*reinterpret_cast<const uint4*>(W + 16 * db * kC + 32 * kk));
  }

  // DMA of block `blk` into stage st: row r (position 64 blk + r) by wave r %
  // 8; lane L fills LDS chunk L of the row from global chunk L ^ (r & 15).
  // Positions past the request or on a page outside the pool read slot 0 and
  // are stored as zeros.
  // (the block's slots and their validity are kept for its stores and rope copy)
  int slot_n = 0;
  uint64_t ok_n = 0;
  auto issue = [&](int blk, int st) {
    const int s = blk * kExpPos + lane;
    const int64_t sl = s < L ? slot_of(b, bi, s) : -1;
    device_check(b, s < L && sl < 0, DSA_CHECK_PAGE_ID);
    const int my_slot = sl < 0 ? 0 : (int)sl;
    slot_n = my_slot;
    ok_n = __ballot(sl >= 0);
#pragma unroll
    for (int i = 0; i < kExpPos / 8; ++i) {
      const int r = wave + 8 * i;
      const int slot = __builtin_amdgcn_readlane(my_slot, r);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(kv + (int64_t)slot * DSA_MLA_DIM), (short)0, DSA_MLA_DIM * 2,
          0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lat[st] + r * kExpRow), 16,
                                               16 * (lane ^ (r & 15)), 0, 0, 0);
    }
  };

  uint16_t* dst = (which ? vn : kn) + ((int64_t)bi * kH + h) * lp * kDn;
  int st = 0;
  issue(share, 0);
  for (int blk = share; blk < nblk; blk += n_share, st ^= 1) {
    const int slot_c = slot_n;   // slot of position 64 blk + lane (0: none)
    const uint64_t ok_c = ok_n;  // bit r: position 64 blk + r is on a page in the pool
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's rows have landed
    __syncthreads();                     // every wave's have; the other stage is free
    if (blk + n_share < nblk) issue(blk + n_share, st ^ 1);
    const unsigned char* T = lat[st];
    v4f acc[2][4];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[db][q] = v4f{0.f, 0.f, 0.f, 0.f};
    // the B operands of k-step kk + 1 are read while kk's products run
    auto read_b = [&](int kk, v8bf (&bf)[4]) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * q + l16;  // r & 15 == l16
        bf[q] = as_frag(*reinterpret_cast<const uint4*>(T + r * kExpRow + 16 * ((4 * kk + g) ^ l16)));
      }
    };
    v8bf bf[2][4];
    read_b(0, bf[0]);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      if (kk + 1 < 16) read_b(kk + 1, bf[(kk + 1) & 1]);
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[db][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[db][kk], bf[kk & 1][q], acc[db][q],
                                                               0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int s = blk * kExpPos + 16 * q + l16;
      const bool ok = (ok_c >> (16 * q + l16)) & 1;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const v4f x = ok ? acc[db][q] : v4f{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<uint2*>(dst + (int64_t)s * kDn + d0 + 16 * db + 4 * g) =
            make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
      }
    }
    if (h == blk % kH) {
      // the rope dims of the block's positions (one head's work-groups per
      // block, spread over the heads), 8 chunks of 16 bytes each
      for (int i = tid; i < kExpPos * 8; i += kExpThreads) {
        const int r = i / 8, c = i % 8;
        const int s = blk * kExpPos + r;
        const int sl = __shfl(slot_c, r);
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if ((ok_c >> r) & 1)
          x = *reinterpret_cast<const uint4*>(kv + (int64_t)sl * DSA_MLA_DIM + kC + 8 * c);
        *reinterpret_cast<uint4*>(rope + ((int64_t)bi * lp + s) * kDr + 8 * c) = x;
      }
    }
  }
}

// ------------------------------------------------------------------ mask
//
// Row t's word w holds positions 32w .. 32w+31: bit set when the row
// attends the position (idx lists it, or idx is NULL and the position is
// visible) and its page is inside the pool.  One work-group per row; the
// listed positions are set in an LDS bitmap first.
constexpr int kMaskThreads = 256;
constexpr int kMaxMaskWords = 2048;  // rows of up to 65536 positions

__global__ __launch_bounds__(kMaskThreads) void mha_mask_kernel(BatchArgs b,
                                                                const int32_t* __restrict__ idx,
                                                                int k, uint32_t* __restrict__ mask,
                                                                int nwords) {
  __shared__ uint32_t bits[kMaxMaskWords];
  const int t = blockIdx.x;
  const int bi = row_request(b.cu, b.B, t);
  const int v = row_visible(b, bi, t);
  for (int w = threadIdx.x; w < nwords; w += kMaskThreads) bits[w] = 0u;
  __syncthreads();
  if (idx) {
    for (int j = threadIdx.x; j < k; j += kMaskThreads) {
      const int s = idx[(int64_t)t * k + j];
      device_check(b, s < -1, DSA_CHECK_INDEX);
      if (s >= 0 && s < v) atomicOr(&bits[s >> 5], 1u << (s & 31));
    }
  } else {
    for (int w = threadIdx.x; w < nwords; w += kMaskThreads) {
      const int lo = 32 * w;
      bits[w] = lo >= v ? 0u : (v - lo >= 32 ? 0xffffffffu : (1u << (v - lo)) - 1u);
    }
  }
  __syncthreads();
  for (int w = threadIdx.x; w < nwords; w += kMaskThreads) {
    uint32_t x = bits[w];
    if (x && slot_of(b, bi, 32 * w) < 0) x = 0u;  // the 32 positions share one page
    mask[(int64_t)t * nwords + w] = x;
  }
}

// ---------------------------------------------------------------- attend
//
// Work-group: 4 waves, 128 consecutive query rows of one request and one
// head; wave w owns rows 32w .. 32w+31 as two blocks of 16.  Key tiles of
// 64 positions pass through LDS, double-buffered, by DMA (buffer loads to LDS):
// K (64 x 128 dims, 16 KB), rope (64 x 64 dims, 8 KB) and V (64 x 128, 16
// KB).  Row chunks are XOR-swizzled so that the operand reads (16 rows at
// one 16-byte column) and the transposing V reads are free of bank
// conflicts: chunk c of K row r sits at chunk c ^ (r & 15) of the row, of V
// row r at c ^ kv_swz(r), of rope row r at c ^ ((r >> 1) & 7).  Per 32-key half tile:
//   S^T   = K Q^T (keys x queries, 6 k-steps of 32 dims: 4 of K, 2 of rope),
//           the wave's queries held in registers as B operands;
//   softmax online per query in fp32, with the mask bits; the reference max
//           is raised only when a score exceeds it by 2^8;
//   O^T  += V^T P^T, P^T straight from the S^T accumulators (bf16), V^T by
//           transposing LDS reads in the token order the accumulators use.
// Each wave owns its queries' outputs (128 dims), so no data crosses waves
// but the K/V tiles.  The loop takes two tiles per pass, one from each stage,
// so that every LDS read is a lane address plus a constant; a left-out key's
// score becomes -inf through a bit select on its mask bit, with no branch.
constexpr int kAttWaves = 4;
constexpr int kAttThreads = 64 * kAttWaves;
constexpr int kQBlk = 32 * kAttWaves;  // query rows per work-group (32 per wave)
constexpr int kKTile = 64;    // keys per tile
constexpr int kKnBytes = kKTile * kDn * 2;   // 16 KB
constexpr int kRBytes = kKTile * kDr * 2;    // 8 KB
constexpr int kVBytes = kKTile * kDn * 2;    // 16 KB
constexpr float kRescaleMargin = 8.f;        // log2 units

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// s_waitcnt immediates (gfx9 encoding): vmcnt(0); lgkmcnt(0)
constexpr unsigned kWaitVmAll = 0x0f70;
constexpr unsigned kWaitLgkmAll = 0xc07f;

// Chunk c (16 bytes) of V row r sits at chunk c ^ kv_swz(r) of the row, of K
// row r at c ^ k_swz(r).  The two-chunk pieces of 8 consecutive rows that
// one half of a transposing V read covers land on distinct chunks under
// kv_swz.  The K operand reads (16 rows at one 16-byte column per 16 lanes,
// the four 16-lane groups at four columns) are conflict-free under r & 15
// and take twice the LDS cycles under kv_swz (measured with a probe of the
// two patterns: 8 against 4 cycles per 16-byte read).
__device__ __forceinline__ int kv_swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int k_swz(int r) { return r & 15; }

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkmAll);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kAttThreads, 2) void mha_attend_kernel(
    BatchArgs b, const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
    const uint16_t* __restrict__ rope, const uint32_t* __restrict__ mask, int nwords, int lp,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse, int nqb) {
  __shared__ __attribute__((aligned(16))) unsigned char Kn[2][kKnBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Rp[2][kRBytes];
  __shared__ __attribute__((aligned(16))) unsigned char Vn[2][kVBytes];

  // XCD x runs heads x, x+8, ...; on each, a head's query blocks back to back
  // (the longest first), so that they share its K and V tiles in L2
  const int xcd = blockIdx.x & 7;
  const int j = blockIdx.x >> 3;
  const int per_head = nqb * b.B;
  const int h = xcd + 8 * (j / per_head);
  if (h >= kH) return;
  const int rem = j % per_head;
  const int bi = rem / nqb;
  const int qb = nqb - 1 - rem % nqb;
  const int c0 = b.cu[bi];
  const int n = b.cu[bi + 1] - c0;
  const int r0 = qb * kQBlk;
  if (r0 >= n) return;
  const int t_last = c0 + min(n, r0 + kQBlk) - 1;
  const int v_max = row_visible(b, bi, t_last);  // rows see more positions as they go
  const int ntiles = (v_max + kKTile - 1) / kKTile;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l16 = lane & 15;
  const int g = lane >> 4;

  // the wave's queries: blocks qi = 0, 1 of 16 rows; lane (l16, g) holds
  // query 16 qi + l16, dims 32 kk + 8 g .. +7 (kk < 4: q_nope, else q_rope)
  int trow[2];
  bool live[2];
  v8bf qf[2][6];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    const int r = r0 + 32 * wave + 16 * qi + l16;
    live[qi] = r < n;
    trow[qi] = c0 + min(r, n - 1);
    const uint16_t* qn = q_nope + ((int64_t)trow[qi] * kH + h) * kDn + 8 * g;
    const uint16_t* qr = q_rope + ((int64_t)trow[qi] * kH + h) * kDr + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[qi][kk] = as_frag(*reinterpret_cast<const uint4*>(qn + 32 * kk));
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      qf[qi][4 + kk] = as_frag(*reinterpret_cast<const uint4*>(qr + 32 * kk));
  }

  // DMA of tile `tile` into stage `st`: 16 + 8 + 16 wave-wide 1 KB loads,
  // 10 per wave.  Load i of K (or V) fills LDS bytes 1024 i .. +1023 = rows
  // 4i .. 4i+3; lane L writes LDS chunk L % 16 of row 4i + L / 16 and so
  // reads global chunk (L % 16) ^ k_swz(row) (K) or (L % 16) ^ kv_swz(row)
  // (V).  Rope load i covers rows 8i .. 8i+7, lane L chunk L % 8 of row 8i +
  // L / 8, from chunk (L % 8) ^ ((row >> 1) & 7).
  const uint16_t* kn_h = kn + ((int64_t)bi * kH + h) * lp * kDn;
  const uint16_t* vn_h = vn + ((int64_t)bi * kH + h) * lp * kDn;
  const uint16_t* rp_b = rope + (int64_t)bi * lp * kDr;
  // A wave's loads are K/V loads i = wave + 4u and rope loads i = wave + 4u -
  // 16: k_swz(row) (K), kv_swz(row) (V) and (row >> 1) & 7 (rope) do not
  // depend on u, so each lane's byte offset within a load's rows is the same
  // for all of them and only the scalar base moves.
  const int kv_row = 4 * wave + (lane >> 4);  // row of the wave's first K/V load
  const uint32_t kn_off = (uint32_t)(kv_row * (kDn * 2) + 16 * ((lane & 15) ^ k_swz(kv_row)));
  const uint32_t kv_off = (uint32_t)(kv_row * (kDn * 2) + 16 * ((lane & 15) ^ kv_swz(kv_row)));
  const int r_row = 8 * wave + (lane >> 3);   // row of the wave's first rope load (mod 32)
  const uint32_t r_off = (uint32_t)((lane >> 3) * (kDr * 2) + 16 * ((lane & 7) ^ ((r_row >> 1) & 7)));
  // buffer resources over the head's K and V rows and the request's rope
  // rows: a tile's loads take a lane offset and a scalar row offset
  const __amdgpu_buffer_rsrc_t kn_r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(kn_h), (short)0, lp * (kDn * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t vn_r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(vn_h), (short)0, lp * (kDn * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rp_r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(rp_b), (short)0, lp * (kDr * 2), 0x00020000);
  auto issue_tile = [&](int tile, int st) {
    const int key0 = tile * kKTile;
#pragma unroll
    for (int u = 0; u < 40 / kAttWaves; ++u) {
      const int i = wave + kAttWaves * u;  // 0..39: K loads 0..15, rope 16..23, V 24..39
      if (i < 16) {
        // rows 4i .. 4i+3: base row 4i - 4 wave (= 4 kAttWaves u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kn_r, (lds_void*)(Kn[st] + 1024 * i), 16, kn_off,
                                                 (key0 + 4 * (i - wave)) * (kDn * 2), 0, 0);
      } else if (i < 24) {
        const int ii = i - 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rp_r, (lds_void*)(Rp[st] + 1024 * ii), 16, r_off,
                                                 (key0 + 8 * ii) * (kDr * 2), 0, 0);
      } else {
        const int ii = i - 24;
        // rows 4 ii .. 4 ii + 3: base row 4 ii - 4 wave
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vn_r, (lds_void*)(Vn[st] + 1024 * ii), 16, kv_off,
                                                 (key0 + 4 * (ii - wave)) * (kDn * 2), 0, 0);
      }
    }
  };

  v4f acc[2][8];  // O^T: [query block][dim block], lane holds dims 16 db + 4 g + r
#pragma unroll
  for (int qi = 0; qi < 2; ++qi)
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[qi][db] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_ref[2] = {-FLT_MAX, -FLT_MAX};
  float l_run[2] = {0.f, 0.f};

  // The mask holds every word of each row (zeros past the row's visible
  // positions), so a lane reads its query's two words of a tile with no
  // test; a lane past the block's end reads the last row's and its results
  // are dropped.
  const uint2* mp[2];
#pragma unroll
  for (int qi = 0; qi < 2; ++qi)
    mp[qi] = reinterpret_cast<const uint2*>(mask + (int64_t)trow[qi] * nwords);
  uint2 mwn[2] = {make_uint2(0u, 0u), make_uint2(0u, 0u)};
  if (ntiles > 0) {
    issue_tile(0, 0);
#pragma unroll
    for (int qi = 0; qi < 2; ++qi) mwn[qi] = mp[qi][0];
  }
  // one tile from stage ST (a constant, so that every LDS read takes an
  // immediate offset on the lane's address)
  auto tile_step = [&](auto st_c, int tile) {
    constexpr int st = decltype(st_c)::value;
    __builtin_amdgcn_s_waitcnt(kWaitVmAll);  // this wave's share of the tile has landed
    lds_barrier();                           // every share has; the other stage is free
    const uint2 mwc[2] = {mwn[0], mwn[1]};
    if (tile + 1 < ntiles) {
      issue_tile(tile + 1, st ^ 1);
#pragma unroll
      for (int qi = 0; qi < 2; ++qi) mwn[qi] = mp[qi][tile + 1];
    }
    const unsigned char* K = Kn[st];
    const unsigned char* R = Rp[st];
    const unsigned char* V = Vn[st];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kb0 = 32 * half;  // first key of the half tile within the tile
      // S^T for both query blocks
      v4f s[2][2];
#pragma unroll
      for (int qi = 0; qi < 2; ++qi) s[qi][0] = s[qi][1] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 6; ++kk) {
        v8bf a[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int row = kb0 + 16 * e + l16;
          if (kk < 4) {
            const int ch = (4 * kk + g) ^ k_swz(row);
            a[e] = as_frag(*reinterpret_cast<const uint4*>(K + row * (kDn * 2) + 16 * ch));
          } else {
            const int ch = (4 * (kk - 4) + g) ^ ((row >> 1) & 7);
            a[e] = as_frag(*reinterpret_cast<const uint4*>(R + row * (kDr * 2) + 16 * ch));
          }
        }
#pragma unroll
        for (int qi = 0; qi < 2; ++qi)
#pragma unroll
          for (int e = 0; e < 2; ++e)
            s[qi][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[e], qf[qi][kk], s[qi][e], 0, 0, 0);
      }
      // softmax; P^T (bf16) for the value product
      uint4 pt[2];
#pragma unroll
      for (int qi = 0; qi < 2; ++qi) {
        // this lane's keys: kb0 + 4 g + r (s[qi][0]) and + 16 (s[qi][1]),
        // bits 4 g + r and 16 + 4 g + r of the half's mask word.  Scores
        // stay unscaled until the exponent (scale_log2 > 0, so the maximum
        // commutes with it); a key left out scores -inf, by a bit select on
        // the mask bit spread over the word.
        const uint32_t mg = (half ? mwc[qi].y : mwc[qi].x) >> (4 * g);
        float z[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t b0 = (uint32_t)((int)(mg << (31 - r)) >> 31);
          const uint32_t b1 = (uint32_t)((int)(mg << (15 - r)) >> 31);
          z[r] = __uint_as_float((__float_as_uint(s[qi][0][r]) & b0) | (0xff800000u & ~b0));
          z[4 + r] = __uint_as_float((__float_as_uint(s[qi][1][r]) & b1) | (0xff800000u & ~b1));
        }
        float tmax = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])),
                           fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
        {
          const v2u x = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax),
                                                         __float_as_uint(tmax), false, false);
          tmax = fmaxf(__uint_as_float(x[0]), __uint_as_float(x[1]));
          const v2u y = __builtin_amdgcn_permlane16_swap(__float_as_uint(tmax),
                                                         __float_as_uint(tmax), false, false);
          tmax = fmaxf(__uint_as_float(y[0]), __uint_as_float(y[1]));
        }
        tmax *= scale_log2;
        // the reference starts at -FLT_MAX (below every finite score): the
        // first finite maximum raises it with a factor of 0 for the empty sums
        if (tmax > m_ref[qi] + kRescaleMargin) {
          const float alpha = __builtin_amdgcn_exp2f(m_ref[qi] - tmax);
          m_ref[qi] = tmax;
          l_run[qi] *= alpha;
#pragma unroll
          for (int db = 0; db < 8; ++db) acc[qi][db] *= alpha;
        }
        float p[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(z[r], scale_log2, -m_ref[qi]));
        l_run[qi] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        pt[qi] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                            pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
      }
      // O^T += V^T P^T: lane (l16, g) takes dim 16 db + l16 of keys 4g .. 4g+3
      // and 16+4g .. 16+4g+3 through transposing reads; lane L of group g
      // addresses key row kb0 + 4g + L/4 (and 16 below) at dims 16 db + 4 (L%4)
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int row = kb0 + 4 * g + (l16 >> 2);
        const int dim = 16 * db + 4 * (l16 & 3);
        const int ch = dim >> 3, sub = (dim & 7) * 2;
        const unsigned char* p_lo = V + row * (kDn * 2) + 16 * (ch ^ kv_swz(row)) + sub;
        const unsigned char* p_hi = V + (row + 16) * (kDn * 2) + 16 * (ch ^ kv_swz(row + 16)) + sub;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p_lo));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p_hi));
        const v8bf va = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qi = 0; qi < 2; ++qi)
          acc[qi][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, as_frag(pt[qi]), acc[qi][db], 0,
                                                                0, 0);
      }
    }
  };
  for (int tile = 0; tile < ntiles; tile += 2) {
    tile_step(std::integral_constant<int, 0>{}, tile);
    if (tile + 1 < ntiles) tile_step(std::integral_constant<int, 1>{}, tile + 1);
  }

#pragma unroll
  for (int qi = 0; qi < 2; ++qi) {
    if (!live[qi]) continue;
    float l_tot = l_run[qi] + __shfl_xor(l_run[qi], 16);
    l_tot += __shfl_xor(l_tot, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* o = out + ((int64_t)trow[qi] * kH + h) * kDn + 4 * g;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const v4f x = acc[qi][db];
      *reinterpret_cast<uint2*>(o + 16 * db) =
          make_uint2(pack_bf16x2(x[0] * inv, x[1] * inv), pack_bf16x2(x[2] * inv, x[3] * inv));
    }
    if (lse && g == 0)
      lse[(int64_t)trow[qi] * kH + h] =
          l_tot > 0.f ? (m_ref[qi] + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

MhaWs mha_ws_layout(const BatchArgs& b) {
  MhaWs w;
  const size_t lp = (size_t)((b.max_seqlen_k + kKTile - 1) / kKTile * kKTile);
  size_t off = 0;
  w.lp = (int)lp;
  w.nwords = (int)(lp / 32);
  w.kn_off = off;
  off += (size_t)b.B * kH * lp * kDn * 2;
  w.vn_off = off;
  off += (size_t)b.B * kH * lp * kDn * 2;
  w.rope_off = off;
  off += (size_t)b.B * lp * kDr * 2;
  w.mask_off = off;
  off += (size_t)b.T * w.nwords * 4;
  w.total = (off + 255) / 256 * 256;
  return w;
}

bool mha_supported(const BatchArgs& b) { return b.max_seqlen_k <= kMaxMaskWords * 32; }

hipError_t launch_masked_mha(const BatchArgs& b, const uint16_t* q_nope, const uint16_t* q_rope,
                             const uint16_t* w_uk, const uint16_t* w_uv, const uint16_t* kv,
                             const int32_t* idx, int k, float sm_scale, uint16_t* out,
                             float* lse, void* ws, hipStream_t s) {
  if (b.T == 0 || b.B == 0) return hipSuccess;
  const MhaWs L = mha_ws_layout(b);
  char* base = static_cast<char*>(ws);
  uint16_t* kn = reinterpret_cast<uint16_t*>(base + L.kn_off);
  uint16_t* vn = reinterpret_cast<uint16_t*>(base + L.vn_off);
  uint16_t* rope = reinterpret_cast<uint16_t*>(base + L.rope_off);
  uint32_t* mask = reinterpret_cast<uint32_t*>(base + L.mask_off);
  if (b.max_seqlen_k > 0) {
    // position shares per request: about one work-group per CU over the
    // batch (each loads its W rows once and streams its share of the
    // latent rows through LDS)
    const int nblk = L.lp / kExpPos;
    const int n_share = std::max(1, std::min(nblk, 256 / (kH * b.B)));
    hipLaunchKernelGGL(mha_expand_kernel, dim3((unsigned)kH, (unsigned)n_share, (unsigned)b.B),
                       dim3(kExpThreads), 0, s, b, kv, w_uk, w_uv, kn, vn, rope, L.lp, n_share);
  }
  hipLaunchKernelGGL(mha_mask_kernel, dim3((unsigned)b.T), dim3(kMaskThreads), 0, s, b, idx, k,
                     mask, L.nwords);
  const int nqb = (b.max_q + kQBlk - 1) / kQBlk;
  hipLaunchKernelGGL(mha_attend_kernel, dim3((unsigned)(8 * (kH / 8) * nqb * b.B)),
                     dim3(kAttThreads), 0, s, b, q_nope, q_rope, kn, vn, rope, mask, L.nwords,
                     L.lp, sm_scale * kLog2e, out, lse, nqb);
  return hipGetLastError();
}

}  // namespace dsa
