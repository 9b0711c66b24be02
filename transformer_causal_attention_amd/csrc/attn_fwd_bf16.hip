// Fused causal attention forward, bf16 in / bf16 out, fp32 accumulation, for gfx950.
//
// What is computed (per batch row b, query head h, query position i, K/V head g = h / G):
//   q' = RoPE(q_i) * log2(e)/sqrt(D)        (in registers, once per row block)
//   s_j = q' . k'_j                          (k' = RoPE(k), produced by the preparation pass)
//   softmax over j <= i in base 2, evaluated online:  out_i = sum_j p_j v_j / sum_j p_j,
//   p_j = 2^(s_j - m), lse_i = ln(2) * (m + log2 sum_j p_j)
// Definitions: scores / sqrt(head_dim), mask of later keys, softmax over keys (llama3-from-
// scratch page: "attention score matrix", "causal mask", "softmax"); the row maximum is
// subtracted before exponentiating (PaLM page, section 2.5); grouped K/V heads (llama3 page,
// "key-value sharing"); the IO-aware, tiled evaluation that never stores the score matrix is
// what the Picotron page calls flash attention ("Flash Attention integration and
// optimisation").
//
// Work decomposition.  A workgroup has 8 waves in two groups of 4 (wave w runs on SIMD w%4,
// so every SIMD holds one wave of each group).  In a group each wave owns 32 query rows of
// one query head; the hpw heads of the group (up to 4 of the G sharing the K/V head) read
// the same K/V tiles, so grouped-query attention stages each tile once per hpw heads.
// Causal work grows linearly with the row block, so a workgroup takes the pair of row blocks
// (r, n-1-r): group A runs all of block r plus the first x key tiles of block n-1-r, group B
// the remaining key tiles of block n-1-r, with x chosen so both groups run the same number of
// tiles; A then hands its partial (max, sum, accumulator) for block n-1-r to B through LDS and
// B merges the two (the same logsumexp merge that joins sequence shards).  Every workgroup
// therefore does the same work, and consecutive workgroup ids walk the (batch, K/V head, head
// group) units so one K/V head stays on one XCD's L2 when the unit count is a multiple of 8.
//
// Data movement.  The preparation pass stores K' and V^T as 64-key tiles in chunk-major order
// ([dimension chunk][key][8] and [key chunk][column][8]).  A tile is copied from HBM straight
// into LDS (global_load_lds, 16 bytes per lane, no registers) as one contiguous run, and every
// MFMA operand is then one 16-byte LDS read at a per-lane base plus a constant offset, with 8
// consecutive lanes reading 128 consecutive bytes (no bank conflicts, no address arithmetic in
// the loop).  K and V^T have two buffers each, in four separate LDS arrays, and the loop is
// unrolled by two, so the compiler can see that operand reads never depend on the copies in
// flight and inserts no wait for them.
//
// Matrix layout.  With A = K tile (32 keys x 16 dims) and B = Q^T (16 dims x 32 rows), the
// 32x32x16 bf16 MFMA yields S^T: lane l holds query row l%32 and, in its 16 accumulators,
// keys 8*(v/4) + 4*(l/32) + v%4.  Row sums are thus in-lane plus one exchange between the lane
// halves at the end.  O^T = V^T P^T takes those accumulators (packed to bf16) as its B operand
// unchanged; the matching A operand (V^T, 8 keys of one column in that order) is one 16-byte
// read, because V^T stores each group of 16 keys in exactly that order.  Keys above the
// diagonal are never loaded, and a wave skips the 32-key blocks entirely above its rows.
//
// Pipeline.  Step i of the loop computes the scores and probabilities of key tile i and the
// P.V product of tile i-1 (whose V^T tile is kept one step longer), so every step has matrix
// work to overlap with the exponentials: QK(b0) | QK(b1) with the exponentials of block 0 |
// the P.V product of the previous tile with the exponentials of block 1.
// The probabilities of a tile wait in registers, packed to bf16, until the next step.
//
// Softmax without a per-tile maximum.  The reference m that probabilities are taken against
// only needs to keep 2^(s - m) finite: the first tile of a row block sets m to its exact row
// maximum (rounded up to a bf16 value), later tiles take their probabilities against m as it
// stands, and a tile is redone (from its scores, still in registers) against max(m, its row
// maximum), with the accumulator and sum rescaled by 2^(m_old - m_new) <= 1, only if some row's
// probability sum passed 2^64 or is not finite.  bf16 and fp32 hold values up to 2^64 with the
// same relative precision as values below 1, and out = o / l, lse = m + log2 l do not depend on
// which m was used.  Because m is a bf16 value, the score product subtracts it itself: one more
// MFMA k-step multiplies a key operand of ones by a query operand of -m.

#include <hip/hip_ext.h>

#include "attn_device.h"

#define LDS_AS __attribute__((address_space(3)))

namespace attn {

constexpr int BN = 64;                      // keys per staged tile
constexpr float kSumLimit = 1.8446744e19f;  // 2^64: above this a tile is redone exactly


__device__ __forceinline__ float xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0] holds lane l%32's value in every lane, r[1] lane 32 + l%32's
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Each lane copies the 16 bytes at byte soff + voff of buffer `rsrc` to lds_base + 16 * lane
// (lds_base and soff wave-uniform, voff = 16 * lane).  Buffer addressing keeps the base in
// scalar registers and the lane offset in one VGPR; reads past the buffer's size return zeros.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, char *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)lds_base, 16, voff, soff, 0, 0);
}

// 16-byte store at byte voff + soff of buffer `rsrc`, written through to device scope (sc1):
// visible to every CU once the store has completed, without a cache write-back.
__device__ __forceinline__ void store_through(const u32x4 &v, __amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, (int)voff, (int)soff, 16);
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N vector memory operations of this wave are outstanding (they complete in
// issue order, so the ones issued before the last N are done).
template <int N>
__device__ __forceinline__ void wait_vm_le() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

__device__ __forceinline__ f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int kReadsAhead = 6;  // LDS operand reads kept in flight ahead of the MFMAs

template <int D, bool CAUSAL, bool DUAL, bool FUSED>
__global__ void __launch_bounds__(512) attn_fwd_bf16_kernel(FwdParams p, RopeTable tab) {
  constexpr int NKK = D / 16;              // MFMA steps over head_dim
  constexpr int NCB = D / 32;              // 32-column blocks of the output
  constexpr int TB = BN * D * 2;           // bytes of one staged K or V^T tile
  constexpr int DMA_PER_WAVE = TB / 4096;  // 1 KiB copies per wave and tile
  // K tiles of even / odd steps and V^T tiles of even / odd steps, each [group][tile]
  __shared__ __attribute__((aligned(1024))) char ldsk0[2 * TB];
  __shared__ __attribute__((aligned(1024))) char ldsk1[2 * TB];
  __shared__ __attribute__((aligned(1024))) char ldsv0[2 * TB];
  __shared__ __attribute__((aligned(1024))) char ldsv1[2 * TB];
  // Rotated queries of group B's row block, handed to group A when A moves on to that block
  // (same rows and heads, wave for wave); before that, the rotation frequencies.
  __shared__ __attribute__((aligned(1024))) char ldsq[4 * NKK * 1024];
  double *freq = reinterpret_cast<double *>(ldsq);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep in SGPRs
  const int grp = wave >> 2;
  const int gw = wave & 3;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work: unit (b, g, head group) and row-block pair.  With DUAL the two groups take two
  // units (2u', 2u'+1) of the same pair and each runs the whole pair of its own unit: for grids
  // with more (unit, pair) items than CUs, one round of workgroups instead of two.
  const int HG = p.G / p.hpw;
  const int u = DUAL ? 2 * (int)(blockIdx.x % (p.n_units / 2)) + grp : (int)(blockIdx.x % p.n_units);
  const int pi = DUAL ? (int)(blockIdx.x / (p.n_units / 2)) : (int)(blockIdx.x / p.n_units);
  const int hg = u % HG;
  const int bg = u / HG;
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;
  const int S = p.S;
  const int RPB = p.rows_per_blk;
  const int r_lo = pi;
  const int r_hi = p.n_row_blocks - 1 - pi;
  // key tiles a row block needs: causal, its last row i sees keys j <= i + delta (delta =
  // q_pos0 - k_pos0, 0 unless the call is one shard of a longer sequence), clamped to [0, S]
  const int delta = p.delta;
  auto n_tiles_of = [&](int r) __attribute__((always_inline)) {
    const int keys = CAUSAL ? max(0, min(S, min(S, (r + 1) * RPB) + delta)) : S;
    return (keys + BN - 1) / BN;
  };
  const int t_lo = n_tiles_of(r_lo);
  const int t_hi = n_tiles_of(r_hi);
  const bool two = r_lo != r_hi;
  // Steps of a group.  Group A: the t_lo tiles of block r_lo (when two), then tiles [0, x) of
  // block r_hi; group B: tiles [x, t_hi) of block r_hi, with x balancing the two.  Inside the
  // loop every update of the accumulators goes through the one tile body (a second one makes
  // the compiler copy them every step): at A's switch the tile of block r_hi's first key tile
  // also adds the P.V product of block r_lo's last one, and the last tile's P.V product is
  // added after the loop.
  // (DUAL: each group runs both blocks of its own unit, as group A with x = t_hi)
  const bool runs_lo = DUAL || grp == 0;
  const int x = DUAL ? t_hi : (two ? (t_hi - t_lo) / 2 : t_hi / 2);  // tiles of block r_hi run by group A
  const int len0 = (runs_lo && two) ? t_lo : 0;
  const int k1s = runs_lo ? 0 : x;
  const int n_mine = len0 + (runs_lo ? x : t_hi - x);
  // rounded up to even (the loop body is two steps; steps after a group's last tile only wait
  // at the barrier)
  const int n_iter = (max((two ? t_lo : 0) + x, t_hi - x) + 1) & ~1;

  const int head = g * p.G + hg * p.hpw + (gw % p.hpw);
  const int sub = gw / p.hpw;

  const size_t n_tiles = (size_t)(p.S_pad / BN);
  const char *kr_tiles = reinterpret_cast<const char *>(p.kr) + ((size_t)b * p.Hkv + g) * n_tiles * TB;
  const char *vt_tiles = reinterpret_cast<const char *>(p.vt) + ((size_t)b * p.Hkv + g) * n_tiles * TB;
  // the K and V^T tiles of this (batch row, K/V head) as buffers (S_pad * D * 2 bytes < 2^31)
  const __amdgpu_buffer_rsrc_t kr_buf = raw_buffer(kr_tiles, (uint32_t)(n_tiles * TB));
  const __amdgpu_buffer_rsrc_t vt_buf = raw_buffer(vt_tiles, (uint32_t)(n_tiles * TB));
  const uint32_t dma_lane = 16u * (uint32_t)lane;

  // per-lane operand bases inside a staged tile (constant parts are immediates):
  //   K of key block jb, step kk:   [chunk 2kk + hh][key 32jb + l32] -> k_lane + 2kk*1024 + jb*512
  //   V^T of block jb, half t, cb:  [chunk 4jb + 2t + hh][column 32cb + l32]
  //                                 -> v_lane + (4jb + 2t)*16*D + cb*512
  const int k_lane = hh * 1024 + l32 * 16;
  const int v_lane = hh * 16 * D + l32 * 16;

  auto tile_of = [&](int i) __attribute__((always_inline)) { return i < len0 ? i : k1s + (i - len0); };
  // this wave's share (DMA_PER_WAVE KiB) of copying tile kt of `buf` to dst
  auto stage = [&](__amdgpu_buffer_rsrc_t buf, int kt, char *dst) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < DMA_PER_WAVE; ++r) {
      const int blk = gw * DMA_PER_WAVE + r;
      lds_dma16(buf, dma_lane, (uint32_t)kt * TB + blk * 1024, dst + blk * 1024);
    }
  };

  // ---- state of this wave's 32 rows
  bf16x8 qf[NKK];
  u32x4 raw_hi[DUAL ? NKK : 1];  // DUAL: block r_hi's queries as loaded, rotated at the switch
  float m_run = 0.f;        // reference the probabilities are taken against (base-2 scores,
                            // always a bf16 value, so that the MFMA below subtracts it exactly)
  // One more k-step of the score product subtracts the reference: row k = 0 of the key operand
  // is 1 and of the query operand -m, so the scores come out as s - m and the exponentials need
  // no subtraction.  Lanes 0-31 hold k = 0..7 of these operands, lanes 32-63 k = 8..15.
  const bf16x8 kaug = __builtin_bit_cast(bf16x8, u32x4{hh ? 0u : 0x3F80u, 0u, 0u, 0u});
  bf16x8 qaug = bf16x8{};
  float l_run = 0.f;        // this lane half's share of the running row sum
  f32x16 o[NCB];
  f32x16 sc0, sc1;          // scores of the tile awaiting its softmax half
  bf16x8 pend[2][2];        // probabilities of the previous tile, [block][key half]; zero if none
  int row0 = 0, cur_seg = -1;
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int t = 0; t < 2; ++t) pend[jb][t] = bf16x8{};
  // ---- row blocks: rows, raw query loads, rotation, fresh state
  auto seg_rows = [&](int seg) __attribute__((always_inline)) {
    row0 = (seg == 0 ? r_lo : r_hi) * RPB + sub * 32;
  };
  // every lane issues the same NKK loads (rows past S load row S-1; clear_dead_q zeroes them
  // once they are in), so a partial wait can count them
  auto load_q = [&](u32x4 (&raw)[NKK]) __attribute__((always_inline)) {
    const int my_row = min(row0 + l32, S - 1);
    if (tab.interleaved) {
      // dims 32kk + 16hh .. +15 of the row; split into evens (raw[kk]) and odds
      // (raw[kk + NKK/2]) by unpair_q once loaded
      const __bf16 *src = p.q + (((size_t)b * S + my_row) * p.Hq + head) * D + 16 * hh;
#pragma unroll
      for (int kk = 0; kk < NKK / 2; ++kk) {
        raw[kk] = *reinterpret_cast<const u32x4 *>(src + 32 * kk);
        raw[kk + NKK / 2] = *reinterpret_cast<const u32x4 *>(src + 32 * kk + 8);
      }
    } else {
      const __bf16 *src = p.q + (((size_t)b * S + my_row) * p.Hq + head) * D + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) raw[kk] = *reinterpret_cast<const u32x4 *>(src + 16 * kk);
    }
  };
  auto clear_dead_q = [&](u32x4 (&raw)[NKK]) __attribute__((always_inline)) {
    if (row0 + l32 >= S) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) raw[kk] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  // adjacent-pair rotary form: the loaded 16-dim runs become the reordered dims (see RopeTable)
  auto unpair_q = [&](u32x4 (&raw)[NKK]) __attribute__((always_inline)) {
    if (tab.interleaved) {
#pragma unroll
      for (int kk = 0; kk < NKK / 2; ++kk) deinterleave16(raw[kk], raw[kk + NKK / 2], raw[kk], raw[kk + NKK / 2]);
    }
  };
  auto rotate_q = [&](const u32x4 (&raw)[NKK]) __attribute__((always_inline)) {
    const int my_row = row0 + l32;
    // rotate pairs (c, c + D/2): lane holds columns 16kk + 8hh + e in raw[kk], kk < NKK/2
#pragma unroll
    for (int kk = 0; kk < NKK / 2; ++kk) {
      u32x4 olo, ohi;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float r[2][2];
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const int e = 2 * w + z;
          const double f = freq[16 * kk + 8 * hh + e];
          const float t = turn_fraction(p.q_pos0 + my_row, f);
          const float sn = __builtin_amdgcn_sinf(t);  // argument in turns
          const float cs = __builtin_amdgcn_cosf(t);
          const uint32_t lo = raw[kk][w], hi = raw[kk + NKK / 2][w];
          const float xv = z ? bf16_hi(lo) : bf16_lo(lo);
          const float yv = z ? bf16_hi(hi) : bf16_lo(hi);
          r[0][z] = (xv * cs - yv * sn) * p.q_scale;
          r[1][z] = (yv * cs + xv * sn) * p.q_scale;
        }
        olo[w] = pack_bf16x2(r[0][0], r[0][1]);
        ohi[w] = pack_bf16x2(r[1][0], r[1][1]);
      }
      qf[kk] = __builtin_bit_cast(bf16x8, olo);
      qf[kk + NKK / 2] = __builtin_bit_cast(bf16x8, ohi);
    }
  };
  // With four heads per group every wave of a group has the same 32 rows, so the workgroup
  // forms each (row, frequency) angle once: a table of (cos, sin) * q_scale for the 32 rows of
  // both row blocks, laid out [block][kk][hh][pair of e][row] x 16 bytes so that a lane's read
  // of its two entries is one 16-byte read and a wave's reads are consecutive.
  // The table sits in a V^T buffer that the first step fills, and is built while the queries
  // are still on their way: the frequencies are loaded before the queries (so waiting for them
  // does not wait for the queries), and the angles only need them and the row positions.
  char *const rot_tab = ldsv0;  // free until step 0 (2 * TB >= 4096 * D / 16 bytes)
  constexpr int TAB_SLOTS = 2 * (NKK / 2) * 2 * 4 * 32;
  constexpr int TAB_FJ = (128 * NKK) / 512;  // distinct frequency sets over a thread's entries
  static_assert(TAB_SLOTS % 512 == 0 && TAB_FJ >= 1, "table entries per thread");
  auto tab_freq_index = [&](int j, int z) __attribute__((always_inline)) {
    const int id = tid + 512 * j;
    const int c = (id / 32) % 4, h2 = (id / 128) % 2, kk = (id / 256) % (NKK / 2);
    return 16 * kk + 8 * h2 + 2 * c + z;
  };
  auto build_rot_tab = [&](const double (&fq)[TAB_FJ][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < TAB_SLOTS / 512; ++j) {
      const int id = tid + 512 * j;
      const int r = id % 32;
      const int s = id / (256 * (NKK / 2));
      const int pos = p.q_pos0 + (s == 0 ? r_lo : r_hi) * RPB + r;
      f32x4 v;
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const float t = turn_fraction(pos, fq[j % TAB_FJ][z]);
        v[2 * z] = __builtin_amdgcn_cosf(t) * p.q_scale;  // argument in turns
        v[2 * z + 1] = __builtin_amdgcn_sinf(t) * p.q_scale;
      }
      *reinterpret_cast<f32x4 *>(rot_tab + id * 16) = v;
    }
  };
  auto rotate_q_tab = [&](const u32x4 (&raw)[NKK], int s) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < NKK / 2; ++kk) {
      u32x4 olo, ohi;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const f32x4 cs = *reinterpret_cast<const f32x4 *>(
            rot_tab + ((((s * (NKK / 2) + kk) * 2 + hh) * 4 + w) * 32 + l32) * 16);
        float r[2][2];
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const uint32_t lo = raw[kk][w], hi = raw[kk + NKK / 2][w];
          const float xv = z ? bf16_hi(lo) : bf16_lo(lo);
          const float yv = z ? bf16_hi(hi) : bf16_lo(hi);
          r[0][z] = xv * cs[2 * z] - yv * cs[2 * z + 1];
          r[1][z] = yv * cs[2 * z] + xv * cs[2 * z + 1];
        }
        olo[w] = pack_bf16x2(r[0][0], r[0][1]);
        ohi[w] = pack_bf16x2(r[1][0], r[1][1]);
      }
      qf[kk] = __builtin_bit_cast(bf16x8, olo);
      qf[kk + NKK / 2] = __builtin_bit_cast(bf16x8, ohi);
    }
  };
  auto set_ref = [&](float m) __attribute__((always_inline)) {  // m: a bf16 value
    m_run = m;
    const uint32_t nm = __float_as_uint(-m) >> 16;
    qaug = __builtin_bit_cast(bf16x8, u32x4{hh ? 0u : nm, 0u, 0u, 0u});
  };
  auto reset_seg = [&]() __attribute__((always_inline)) {
    // the first tile of a row block always takes the exact maximum, which replaces this
    // provisional reference before any probability is kept
    set_ref(0.f);
    l_run = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{};
  };
  // the hand-off slot of wave gw: NKK rows of 64 lanes x 16 bytes (the lane offset is made
  // opaque where it is used, so no address is kept live across the loop)
  auto q_slot = [&]() __attribute__((always_inline)) {
    uint32_t lo = dma_lane;
    asm volatile("" : "+v"(lo));
    return ldsq + gw * NKK * 1024 + lo;
  };

  // out and lse of the rows starting at r0 from o, this lane half's sum l_half and reference m
  auto store_seg = [&](int r0, float l_half, float m) __attribute__((always_inline)) {
    const float l_tot = l_half + xor32(l_half);
    // lane indices made opaque, so no per-lane part of the addresses is kept live across the loop
    int lr = l32, lh = hh;
    asm volatile("" : "+v"(lr), "+v"(lh));
    const int my_row = r0 + lr;
    if (my_row < S) {
      // a row with no visible key (possible only in a shard of later keys) has out 0, lse -inf
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
      __bf16 *dst = p.out + (((size_t)b * S + my_row) * p.Hq + head) * D + 4 * lh;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          u32x2 w2;
          w2[0] = pack_bf16x2(o[cb][4 * a + 0] * inv, o[cb][4 * a + 1] * inv);
          w2[1] = pack_bf16x2(o[cb][4 * a + 2] * inv, o[cb][4 * a + 3] * inv);
          *reinterpret_cast<u32x2 *>(dst + 32 * cb + 8 * a) = w2;
        }
      if (lh == 0)
        p.lse[((size_t)b * p.Hq + head) * S + my_row] =
            l_tot > 0.f ? (m + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
  };

  // ---- block pieces (kd / vd: this group's K and V^T tile)
  auto kfrag = [&](const char *kd, int jb, int kk) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8 *>(kd + k_lane + 2 * kk * 1024 + jb * 512);
  };
  auto vfrag = [&](const char *vd, int jb, int t, int cb) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8 *>(vd + v_lane + (4 * jb + 2 * t) * 16 * D + cb * 512);
  };
  constexpr int NPV = 4 * NCB;            // MFMAs of the P.V product of one tile
  constexpr int NMF = 2 * NKK + NPV;      // MFMAs of one tile
  constexpr int NDMA = 2 * DMA_PER_WAVE;  // copy instructions per step of a wave (its group's two tiles)
  static_assert(3 * (NDMA - 1) < NMF, "every copy is issued inside the tile");
  auto pv_of = [&](const char *vd, int r) __attribute__((always_inline)) {  // operand of the r-th P.V MFMA
    const int jb = r / (2 * NCB), t = (r / NCB) % 2, cb = r % NCB;
    return vfrag(vd, jb, t, cb);
  };
  // keys after the query or past the sequence end get -inf (only called where some may be)
  auto mask = [&](f32x16 &sc, int kb0) __attribute__((always_inline)) {
    const int my_row = row0 + l32;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = kb0 + 8 * (v >> 2) + 4 * hh + (v & 3);
      if ((CAUSAL && j > my_row + delta) || j >= S) sc[v] = -INFINITY;
    }
  };
  auto needs_redo = [&](float rsum) __attribute__((always_inline)) {
    return __builtin_amdgcn_ballot_w64(!(rsum <= kSumLimit)) != 0;  // also catches inf and NaN
  };
  // The two tile copies of a step for a group (its next K tile and this step's V^T tile); the
  // group's waves move their share of each, one instruction at a time between softmax work.
  struct Copies {
    int tile[2];  // K tile, V^T tile
    char *dst[2];
  };
  auto copy_part = [&](const Copies &c, int r) __attribute__((always_inline)) {
    const int q = r / DMA_PER_WAVE;
    const int blk = gw * DMA_PER_WAVE + r % DMA_PER_WAVE;
    lds_dma16((q & 1) ? vt_buf : kr_buf, dma_lane, (uint32_t)c.tile[q] * TB + blk * 1024, c.dst[q] + blk * 1024);
  };

  // ---- one key tile per step: QK(b0) | QK(b1) with the probabilities of block 0 | P.V of the
  // previous tile with the probabilities of block 1, operand reads kReadsAhead MFMAs ahead, one
  // fenced unit per MFMA so the issue order is the one written here.  The probabilities are
  // taken against m as it stands; the 16 pairs of scores (8 per block) go through two stages a
  // pair apart (exponentials of pair w; packing of pair w-1 to bf16 and its addition to the row
  // sums), so no instruction waits on the one before it.  Row sums use plain VALU adds: the
  // bf16 dot-product instruction would queue behind MFMAs.  Each wave also issues its share
  // of its group's copies for the step (the next K tile, this step's V^T tile), one every third
  // MFMA from the first, so the last copy has a third of the tile to land before the step's
  // wait.  Afterwards the tile is redone against its exact maximum when it is the first of its
  // row block or a row's sum passed the limit, from the scores still in registers.
  auto tile = [&](const char *kd, const char *vd, int kb0, bool msk, bool first, bool issue,
                  const Copies &cp) __attribute__((always_inline)) {
    auto op_of = [&](int g) __attribute__((always_inline)) {
      return g < NKK ? kfrag(kd, 0, g) : g < 2 * NKK ? kfrag(kd, 1, g - NKK) : pv_of(vd, g - 2 * NKK);
    };
    bf16x8 fr[kReadsAhead];
#pragma unroll
    for (int r = 0; r < kReadsAhead; ++r) fr[r] = op_of(r);
    auto unit_tail = [&](int g) __attribute__((always_inline)) {
      if (g + kReadsAhead < NMF) fr[g % kReadsAhead] = op_of(g + kReadsAhead);
      if (g % 3 == 0 && g / 3 < NDMA && issue) copy_part(cp, g / 3);
    };
    u32x4 pw0[2], pw1[2];
    float rsum[4];
    float ex0 = 0.f, ex1 = 0.f;  // exponentials of the pair in flight
    float rs0 = 0.f, rs1 = 0.f;
    auto sc_of = [&](int w, int e) __attribute__((always_inline)) {
      return w < 8 ? sc0[2 * w + e] : sc1[2 * (w - 8) + e];
    };
    // scores are s - m already; the exact path subtracts the change of reference sh
    auto pair_stage = [&](int w, float sh, bool shifted) __attribute__((always_inline)) {  // w = 0 .. 16
      if (w >= 1) {  // pair w-1: packed to bf16, added to its row sums
        const int c = w - 1;
        const uint32_t pk = pack_bf16x2(ex0, ex1);
        if (c < 8)
          pw0[c >> 2][c & 3] = pk;
        else
          pw1[(c - 8) >> 2][(c - 8) & 3] = pk;
        rsum[2 * (c >> 3)] += ex0;
        rsum[2 * (c >> 3) + 1] += ex1;
      }
      if (w <= 15) {  // pair w: exponentials
        ex0 = __builtin_amdgcn_exp2f(shifted ? sc_of(w, 0) - sh : sc_of(w, 0));
        ex1 = __builtin_amdgcn_exp2f(shifted ? sc_of(w, 1) - sh : sc_of(w, 1));
      }
    };
    auto pin = [&]() __attribute__((always_inline)) {
      // consumed here, so each unit's share of the pipeline stays in its place
      asm volatile("" ::"v"(ex0), "v"(ex1), "v"(rsum[0]), "v"(rsum[1]), "v"(rsum[2]), "v"(rsum[3]));
    };
#pragma unroll
    for (int r = 0; r < 4; ++r) rsum[r] = 0.f;
    // phase 1: QK(b0), starting from -m
    sc0 = mfma(kaug, qaug, f32x16{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      sc0 = mfma(fr[kk % kReadsAhead], qf[kk], sc0);
      unit_tail(kk);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (msk) mask(sc0, kb0);
    __builtin_amdgcn_sched_barrier(0);
    // phase 2: QK(b1), starting from -m, with the probabilities of block 0
    sc1 = mfma(kaug, qaug, f32x16{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int g = NKK + kk;
      sc1 = mfma(fr[g % kReadsAhead], qf[kk], sc1);
      unit_tail(g);
#pragma unroll
      for (int w = kk * 8 / NKK; w < (kk + 1) * 8 / NKK; ++w) pair_stage(w, 0.f, false);
      pin();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (msk) mask(sc1, kb0 + 32);
    __builtin_amdgcn_sched_barrier(0);
    // phase 3: P.V of the previous tile with the probabilities of block 1
#pragma unroll
    for (int r = 0; r < NPV; ++r) {
      const int g = 2 * NKK + r;
      const int jb = r / (2 * NCB), t = (r / NCB) % 2, cb = r % NCB;
      o[cb] = mfma(fr[g % kReadsAhead], pend[jb][t], o[cb]);
      unit_tail(g);
#pragma unroll
      for (int w = 8 + r * 9 / NPV; w < 8 + (r + 1) * 9 / NPV; ++w) pair_stage(w, 0.f, false);
      pin();
      __builtin_amdgcn_sched_barrier(0);
    }
    rs0 = rsum[0] + rsum[1];
    rs1 = rsum[2] + rsum[3];
    if (first || needs_redo(rs0 + rs1)) {
      float mx = fmaxf(sc0[0], sc1[0]);
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(sc0[v], sc1[v]));
      mx = max_xor32(mx);
      // mx is the row maximum of s - m.  The first tile of a row block replaces the provisional
      // reference (its state is still empty, so nothing is rescaled); later the reference only
      // grows, so every rescale factor is at most 1.  A row with no visible key keeps its
      // reference.  The new reference is rounded up to a bf16 value, so every probability is at
      // most 1 and the largest ones keep bf16's finest relative spacing below 1.
      const float m_abs = first ? (mx == -INFINITY ? m_run : m_run + mx) : m_run + fmaxf(0.f, mx);
      const uint32_t mb = __float_as_uint(m_abs);
      const float m_new = __uint_as_float(m_abs > 0.f ? (mb + 0xFFFFu) & 0xFFFF0000u : mb & 0xFFFF0000u);
      const float d = m_new - m_run;  // the change of reference (>= 0 unless first)
      const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(-d);
      // (o is zero at a row block's first tile, or at group A's switch block r_lo's
      // accumulator, which is kept as is)
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
      set_ref(m_new);
#pragma unroll
      for (int r = 0; r < 4; ++r) rsum[r] = 0.f;
#pragma unroll
      for (int w = 0; w <= 16; ++w) pair_stage(w, d, true);
      rs0 = rsum[0] + rsum[1];
      rs1 = rsum[2] + rsum[3];
    }
    l_run += rs0 + rs1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pend[0][t] = __builtin_bit_cast(bf16x8, pw0[t]);
      pend[1][t] = __builtin_bit_cast(bf16x8, pw1[t]);
    }
  };

  // ---- main loop.  Step i: K tile i in ldsk[i%2], V^T tile i-1 in ldsv[(i+1)%2]; the copies
  // of K tile i+1 into ldsk[(i+1)%2] and V^T tile i into ldsv[i%2], issued by the tile, run
  // meanwhile.  Unrolled by two so the buffer of every access is known at compile time.
  auto step = [&](int i, const char *kcur, char *knxt, const char *vprev, char *vfill) __attribute__((always_inline)) {
    const int go = grp * TB;
    // this group's copies: K tile i+1 and V^T tile i (an index past the group's last tile is
    // clamped to it: an in-bounds duplicate into a buffer the group no longer reads)
    Copies cp;
    cp.tile[0] = tile_of(max(min(i + 1, n_mine - 1), 0));
    cp.dst[0] = knxt + go;
    cp.tile[1] = tile_of(max(min(i, n_mine - 1), 0));
    cp.dst[1] = vfill + go;
    if (i < n_mine) {
      // group A's switch: this tile is block r_hi's first, its P.V product block r_lo's last;
      // r_lo's sum and reference are kept aside until that product is in o
      const bool sw_now = i == len0 && len0 > 0;
      float l_lo = 0.f, m_lo = 0.f;
      if (sw_now) {
        l_lo = l_run;
        m_lo = m_run;
        seg_rows(1);
        if constexpr (DUAL) {
          clear_dead_q(raw_hi);
          unpair_q(raw_hi);
          rotate_q(raw_hi);
        } else {
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8 *>(q_slot() + kk * 1024);
        }
        l_run = 0.f;
        set_ref(0.f);  // provisional, replaced by the first tile's exact maximum
        cur_seg = 1;
      }
      const int kb0 = tile_of(i) * BN;
      const bool msk = (CAUSAL && kb0 + BN - 1 > row0 + delta) || kb0 + BN > S;
      tile(kcur + go, vprev + go, kb0, msk, i == 0 || i == len0, true, cp);
      if (sw_now) {
        store_seg(r_lo * RPB + sub * 32, l_lo, m_lo);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{};
      }
    }
    wait_vm_all();
    __syncthreads();
  };

  // ---- one-launch form (FUSED): before attending, each wave group prepares some 64-key
  // tiles of its (batch row, K/V head) -- the work of the separate preparation pass, spread
  // over the workgroups that read those tiles -- and publishes them, then waits until every
  // tile its workgroup reads is published.  A job is one half of a tile: the rotated keys
  // (rotary embedding of k at positions k_pos0 + j, half-split pairs (c, c + D/2) after the
  // adjacent-pair reordering when that form is chosen: Picotron page section 1, PaLM page
  // 2.3) or the values transposed into the V^T layout.  Worker w of a (b, g) does jobs
  // w, w + prep_workers, ...  The tiles are stored with device-scope write-through stores, and
  // a half's flag gets this call's tag (a device-scope store) once every wave's stores have
  // completed; the waiting wave reads the flags at device scope.  No cache can hold an older
  // copy of a tile: caches start each kernel without stale lines of memory other kernels
  // wrote, and no workgroup reads a tile before its flags carry the tag, so the staging
  // copies that follow see the tiles.  This avoids a write-back and an invalidation of a
  // whole L2 per workgroup, which a release/acquire pair at device scope would cost.  Every
  // workgroup of the grid is resident at once (the host launches this form only then), so
  // the wait ends; it is bounded all the same, and a workgroup whose wait runs out records
  // kStatusTimeout and writes NaN to its rows.
  constexpr int NL = D / 32;  // 16-byte loads per thread and preparation job (either half)
  const int prep_tid = tid & 255;
  const int prep_worker = DUAL ? pi * HG + hg : (pi * HG + hg) * 2 + grp;
  const int prep_jobs = 2 * (int)n_tiles;
  const size_t rs = (size_t)p.Hkv * D;  // elements between consecutive keys in k, v
  char *const vstage = ldsk1 + grp * TB;  // a group's staged values: [64 keys][D] bf16
  // the loads of round rnd's job, the same NL loads for either half and without branches (a
  // thread without a job loads the keys of tile 0 and ignores them), so that they stay in
  // flight behind the query loads
  //   keys:   item (key row = lane, chunk pair cp = gw + 4 * (i / 2)); chunk pair cp holds dims
  //           8cp.. and D/2 + 8cp.. (adjacent-pair form: 16cp..16cp+15, split into evens and
  //           odds once loaded)
  //   values: item (key row, 8-dim chunk) = prep_tid + 256 * i
  //   rows past S load row S-1 and are zeroed once loaded
  auto prep_load = [&](int rnd, u32x4 (&ld)[NL]) __attribute__((always_inline)) {
    const int job_r = prep_worker + rnd * p.prep_workers;
    const int job = job_r < prep_jobs ? job_r : 0;
    const bool is_v = (job & 1) != 0;
    const int j0 = (job >> 1) * BN;
    const __bf16 *base = (is_v ? p.v : p.k) + (size_t)b * S * rs + (size_t)g * D;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int item = prep_tid + 256 * i;
      const int cp = gw + 4 * (i / 2);
      const int kcol = tab.interleaved ? 16 * cp + 8 * (i & 1) : 8 * cp + (i & 1) * (D / 2);
      const int row = is_v ? item / (D / 8) : lane;
      const int col = is_v ? 8 * (item % (D / 8)) : kcol;
      ld[i] = *reinterpret_cast<const u32x4 *>(base + (size_t)min(j0 + row, S - 1) * rs + col);
    }
  };
  // once the loads are in: keys rotated and stored; values staged in LDS
  auto prep_work_a = [&](int rnd, const u32x4 (&ld)[NL]) __attribute__((always_inline)) {
    const int job = prep_worker + rnd * p.prep_workers;
    if (job >= prep_jobs) return;
    const int j0 = (job >> 1) * BN;
    const uint32_t tile_off = (uint32_t)(job >> 1) * TB;  // in this (b, g)'s run of tiles
    if ((job & 1) == 0) {
#pragma unroll
      for (int it = 0; it < NL / 2; ++it) {
        const int cp = gw + 4 * it;
        const int j = j0 + lane;
        u32x4 xk = ld[2 * it], yk = ld[2 * it + 1];
        if (tab.interleaved) deinterleave16(ld[2 * it], ld[2 * it + 1], xk, yk);
        u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
        if (j < S) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float t0 = turn_fraction(p.k_pos0 + j, tab.rev[8 * cp + 2 * w]);
            const float t1 = turn_fraction(p.k_pos0 + j, tab.rev[8 * cp + 2 * w + 1]);
            // (hardware sin/cos take turns)
            const u32x2 r = rotate_packed(xk[w], yk[w], __builtin_amdgcn_cosf(t0), __builtin_amdgcn_sinf(t0),
                                          __builtin_amdgcn_cosf(t1), __builtin_amdgcn_sinf(t1));
            lo[w] = r[0];
            hi[w] = r[1];
          }
        }
        store_through(lo, kr_buf, dma_lane, tile_off + cp * 1024);
        store_through(hi, kr_buf, dma_lane, tile_off + (cp + D / 16) * 1024);
      }
    } else {
#pragma unroll
      for (int it = 0; it < NL; ++it) {
        const int item = prep_tid + 256 * it;
        const int row = item / (D / 8), ch = item % (D / 8);
        *reinterpret_cast<u32x4 *>(vstage + row * (D * 2) + ch * 16) = j0 + row < S ? ld[it] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  // after a barrier: the staged values leave as the V^T tile, [8 key chunks qq][D columns c][8
  // keys]; inside each group of 16 keys the key at position p0 is swap23(p0) (bits 2 and 3
  // exchanged), the order in which the score accumulators list their keys
  auto prep_work_b = [&](int rnd) __attribute__((always_inline)) {
    const int job = prep_worker + rnd * p.prep_workers;
    if (job >= prep_jobs || (job & 1) == 0) return;
    const uint32_t tile_off = (uint32_t)(job >> 1) * TB;
    const uint16_t *vs = reinterpret_cast<const uint16_t *>(vstage);
#pragma unroll
    for (int it = 0; it < NL; ++it) {
      const int item = prep_tid + 256 * it;
      const int c = item % D, qq = item / D;
      u32x4 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p0 = 8 * qq + 2 * e;
        const int r0 = (p0 & ~12) | ((p0 & 4) << 1) | ((p0 & 8) >> 1);
        w4[e] = (uint32_t)vs[r0 * D + c] | ((uint32_t)vs[(r0 + 1) * D + c] << 16);
      }
      store_through(w4, vt_buf, 16u * (uint32_t)c, tile_off + qq * (D * 16));
    }
  };
  // publish: the tiles were written through to device scope, and every wave's stores have
  // completed before the barrier; one thread per group then tags the halves its group wrote
  auto publish = [&]() __attribute__((always_inline)) {
    wait_vm_all();
    __syncthreads();
    if (prep_tid == 0) {
      const size_t bg_id = (size_t)b * p.Hkv + g;
      for (int rnd = 0; rnd < p.prep_rounds; ++rnd) {
        const int job = prep_worker + rnd * p.prep_workers;
        if (job < prep_jobs)
          __hip_atomic_store(p.flags + bg_id * n_tiles * 2 + job, p.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  // wait: one wave per (b, g) the workgroup reads (both groups share it unless DUAL) checks
  // both halves of tiles 0 .. t_hi-1, the tiles any of its rows can see
  auto await_tiles = [&]() __attribute__((always_inline)) -> bool {
    const size_t bg_id = (size_t)b * p.Hkv + g;
    int *const verdict = reinterpret_cast<int *>(ldsk1);  // [group]
    if (gw == 0 && (DUAL || grp == 0)) {
      const unsigned long long *fl = p.flags + bg_id * n_tiles * 2;
      const int n_fl = 2 * t_hi;
      bool ok = false;
      for (int poll = 0; poll < p.max_polls; ++poll) {
        bool mine = true;
        for (int f = lane; f < n_fl; f += 64)
          mine = mine && __hip_atomic_load(fl + f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == p.await_tag;
        if (__builtin_amdgcn_ballot_w64(!mine) == 0) {
          ok = true;
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
      if (!ok && lane == 0) __hip_atomic_store(p.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0) verdict[grp] = ok ? 1 : 0;
    }
    __syncthreads();
    const bool ok = DUAL ? (verdict[0] & verdict[1]) != 0 : verdict[0] != 0;
    __syncthreads();  // the verdict is read before anything is copied into ldsk1
    return ok;
  };
  // a workgroup that gave up waiting writes NaN to every row it owns
  auto fail_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{} + __builtin_nanf("");
    // (a positive sum with a NaN reference makes both out and lse NaN)
    if (runs_lo && two) store_seg(r_lo * RPB + sub * 32, 1.f, __builtin_nanf(""));
    if (DUAL || grp == 1) store_seg(r_hi * RPB + sub * 32, 1.f, __builtin_nanf(""));
  };

  // ---- prologue: the first row block's queries are loaded while the first K tile is copied,
  // then rotated; group B leaves its rotated queries in its hand-off slot for group A (read at
  // A's switch to block r_hi, at step len0 >= 1, so after at least one barrier).  The P.V
  // product of a step always runs; with zero probabilities it must read finite values, so the
  // V^T buffer that step 0 reads starts out zeroed (later the V^T buffers only ever hold
  // staged tiles).
  {
    seg_rows(len0 > 0 ? 0 : 1);
    cur_seg = n_mine > 0 ? (len0 > 0 ? 0 : 1) : -1;
    const bool shared_tab = p.hpw == 4;
    double fq[TAB_FJ][2];
    if (shared_tab) {
#pragma unroll
      for (int j = 0; j < TAB_FJ; ++j)
#pragma unroll
        for (int z = 0; z < 2; ++z) fq[j][z] = tab.rev[tab_freq_index(j, z)];
    }
    // this thread's rotation frequency for the LDS copy (DUAL, or fewer than four heads per
    // group), loaded unconditionally so that no branch waits for it here
    const double fr_own = tab.rev[min(tid, D / 2 - 1)];
    u32x4 raw[NKK];
    u32x4 ld[NL];
    // one-launch form: the preparation job's loads go first, so its tiles are published as
    // early as possible (every workgroup of the (b, g) waits for the last of them)
    if constexpr (FUSED) prep_load(0, ld);
    if constexpr (DUAL) {
      if (len0 > 0) {  // block r_hi's queries come in now and wait in registers for the switch
        seg_rows(1);
        load_q(raw_hi);
        seg_rows(0);
      }
    }
    load_q(raw);
    if constexpr (!FUSED) {
      if (n_mine > 0) stage(kr_buf, tile_of(0), ldsk0 + grp * TB);  // first K tile of each group
    }
    {
      u32x4 *z1 = reinterpret_cast<u32x4 *>(ldsv1);
#pragma unroll
      for (int r = 0; r < 2 * TB / 16 / 512; ++r) z1[tid + 512 * r] = u32x4{0u, 0u, 0u, 0u};
    }
    // (DUAL keeps the frequencies in LDS for the rotation at the switch: no hand-off slot)
    if (DUAL || !shared_tab) {
      if (tid < D / 2) freq[tid] = fr_own;
    }
    if (shared_tab) build_rot_tab(fq);
    if constexpr (FUSED) {
      // the job's loads are in once at most the query loads issued after them are outstanding
      if (DUAL && len0 > 0)
        wait_vm_le<2 * NKK>();
      else
        wait_vm_le<NKK>();
      prep_work_a(0, ld);
      __syncthreads();
      prep_work_b(0);
      __syncthreads();
      for (int rnd = 1; rnd < p.prep_rounds; ++rnd) {  // the same count in every group
        prep_load(rnd, ld);
        wait_vm_all();
        prep_work_a(rnd, ld);
        __syncthreads();
        prep_work_b(rnd);
        __syncthreads();
      }
      publish();  // waits for every load and store of the wave, then a barrier
    } else {
      wait_vm_all();
      __syncthreads();
    }
    clear_dead_q(raw);
    unpair_q(raw);
    if (shared_tab)
      rotate_q_tab(raw, len0 > 0 ? 0 : 1);
    else
      rotate_q(raw);
    // the frequencies (in the hand-off slot unless DUAL) are no longer read
    __syncthreads();
    if constexpr (FUSED) {
      if (!await_tiles()) {
        fail_rows();
        return;  // uniform over the workgroup: no barrier follows for anyone
      }
      if (n_mine > 0) stage(kr_buf, tile_of(0), ldsk0 + grp * TB);  // first K tile of each group
      wait_vm_all();  // (made visible to every wave by the barrier closing the prologue)
    }
    reset_seg();
    // block r_lo sees no key at all (a shard of later keys): its rows are empty
    if (runs_lo && two && t_lo == 0) store_seg(r_lo * RPB + sub * 32, 0.f, 0.f);
    if (!DUAL && grp == 1) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) *reinterpret_cast<bf16x8 *>(q_slot() + kk * 1024) = qf[kk];
    }
    __syncthreads();  // the table is no longer read before step 0 copies into its buffer
  }
  for (int i = 0; i < n_iter; i += 2) {
    step(i, ldsk0, ldsk1, ldsv1, ldsv0);
    step(i + 1, ldsk1, ldsk0, ldsv0, ldsv1);
  }
  // the last tile's P.V product (its V^T tile went to ldsv[(n_mine - 1) % 2])
  if (n_mine > 0) {
    const char *vd = (((n_mine - 1) & 1) ? ldsv1 : ldsv0) + grp * TB;
#pragma unroll
    for (int r = 0; r < NPV; ++r) {
      const int jb = r / (2 * NCB), t = (r / NCB) % 2, cb = r % NCB;
      o[cb] = mfma(vfrag(vd, jb, t, cb), pend[jb][t], o[cb]);
    }
    if (cur_seg == 0) store_seg(row0, l_run, m_run);  // r_lo was group A's only block (r_hi is merged below)
  }

  // ---- finish: the split block r_hi is merged in B.  Once every wave's last P.V product is
  // done the tile buffers are free: per-wave accumulators of group A go to ldsk0 (waves 0, 1)
  // and ldsk1 (waves 2, 3), maxima and sums to ldsv0; B's finished rows go to ldsv1.
  __syncthreads();  // every wave's last P.V product has read its V^T tile
  if (!DUAL && x > 0) {
    float *mo = reinterpret_cast<float *>(gw < 2 ? ldsk0 : ldsk1) + (gw & 1) * NCB * 16 * 64;
    float *mm = reinterpret_cast<float *>(ldsv0);
    // accumulators as [cb][v / 4][lane][v % 4]: one 16-byte access per lane and 4 registers
    f32x4 *mo4 = reinterpret_cast<f32x4 *>(mo);
    if (grp == 0) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          mo4[(cb * 4 + v4) * 64 + lane] = f32x4{o[cb][4 * v4], o[cb][4 * v4 + 1], o[cb][4 * v4 + 2], o[cb][4 * v4 + 3]};
      mm[gw * 64 + lane] = m_run;
      mm[256 + gw * 64 + lane] = l_run;
    }
    __syncthreads();
    if (grp == 1) {
      const float ma = mm[gw * 64 + lane];
      const float la = mm[256 + gw * 64 + lane];
      // a part in which a row saw no key (sum 0 over both lane halves; only in a shard of
      // later keys) holds a provisional reference only and must not set the merged one
      const float ma_e = la + mm[256 + gw * 64 + (lane ^ 32)] > 0.f ? ma : -INFINITY;
      const float mb_e = l_run + xor32(l_run) > 0.f ? m_run : -INFINITY;
      const float m_max = fmaxf(ma_e, mb_e);
      const float m_new = m_max == -INFINITY ? 0.f : m_max;  // both parts empty: sum stays 0
      const float ca = __builtin_amdgcn_exp2f(ma_e - m_new);
      const float cb_ = __builtin_amdgcn_exp2f(mb_e - m_new);
      l_run = la * ca + l_run * cb_;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x4 a4 = mo4[(cb * 4 + v4) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[cb][4 * v4 + e] = a4[e] * ca + o[cb][4 * v4 + e] * cb_;
        }
      m_run = m_new;
    }
  }
  // Group B's rows of block r_hi (with DUAL both groups' rows, A's in ldsv0) leave through
  // LDS: each wave writes its 32 rows x D output (bf16) to ldsv1 as rows of D / 8 16-byte chunks,
  // chunk c of row r at position c ^ (r % (D / 8)) (so a store instruction's 32 rows spread over
  // the banks), and then all eight waves copy whole rows to HBM with 16-byte stores, D * 2
  // contiguous bytes per (row, head).
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int WB = 32 * D * 2;    // staged bytes per wave
  if (DUAL || grp == 1) {
    const float l_tot = l_run + xor32(l_run);
    const int my_row = row0 + l32;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;  // a row with no visible key: out 0
    char *st = (grp ? ldsv1 : ldsv0) + gw * WB + l32 * (D * 2) + 8 * hh;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 w2;
        w2[0] = pack_bf16x2(o[cb][4 * a + 0] * inv, o[cb][4 * a + 1] * inv);
        w2[1] = pack_bf16x2(o[cb][4 * a + 2] * inv, o[cb][4 * a + 3] * inv);
        *reinterpret_cast<u32x2 *>(st + (((4 * cb + a) ^ (l32 % CPR)) * 16)) = w2;
      }
    if (hh == 0 && my_row < S)
      p.lse[((size_t)b * p.Hq + head) * S + my_row] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
  __syncthreads();
#pragma unroll
  for (int sg = DUAL ? 0 : 1; sg < 2; ++sg) {  // staged group: its unit, buffer and rows
    const int su = DUAL ? 2 * (int)(blockIdx.x % (p.n_units / 2)) + sg : u;
    const int shg = su % HG, sbg = su / HG;
    const int sgk = sbg % p.Hkv, sb = sbg / p.Hkv;
    const char *sbuf = sg ? ldsv1 : ldsv0;
#pragma unroll
    for (int k = 0; k < 16 * D / 512; ++k) {
      const int c = tid + 512 * k;      // chunk of the 4 staged waves' rows
      const int w = c / (4 * D), r = (c % (4 * D)) / CPR, ch = c % CPR;
      const int row = r_hi * RPB + (w / p.hpw) * 32 + r;
      const int hd = sgk * p.G + shg * p.hpw + (w % p.hpw);
      const u32x4 val = *reinterpret_cast<const u32x4 *>(sbuf + w * WB + r * (D * 2) + ((ch ^ (r % CPR)) * 16));
      if (row < S) *reinterpret_cast<u32x4 *>(p.out + (((size_t)sb * S + row) * p.Hq + hd) * D + 8 * ch) = val;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_attn_bf16(const FwdParams &p, const RopeTable &tab, hipStream_t stream,
                            hipEvent_t ev_start, hipEvent_t ev_stop) {
  const bool fused = p.flags != nullptr;
  if constexpr (D == 64) {
    if (p.dual) {  // two units per workgroup (the host checks that n_units is even)
      const long long blocks = (long long)(p.n_units / 2) * p.n_pairs;
      if (fused)
        hipExtLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, true, true>), dim3((unsigned)blocks), dim3(512), 0,
                              stream, ev_start, ev_stop, 0, p, tab);
      else
        hipExtLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, true, false>), dim3((unsigned)blocks), dim3(512), 0,
                              stream, ev_start, ev_stop, 0, p, tab);
      return hipGetLastError();
    }
  }
  const long long blocks = (long long)p.n_units * p.n_pairs;
  if (fused)
    hipExtLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, false, true>), dim3((unsigned)blocks), dim3(512), 0, stream,
                          ev_start, ev_stop, 0, p, tab);
  else
    hipExtLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, false, false>), dim3((unsigned)blocks), dim3(512), 0,
                          stream, ev_start, ev_stop, 0, p, tab);
  return hipGetLastError();
}

// Workgroups of the forward kernel that one CU holds at once (the one-launch form needs the
// whole grid resident).
template <int D>
int fwd_bf16_wgs_per_cu(bool dual) {
  int n = 0;
  hipError_t e;
  if (D == 64 && dual)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_fwd_bf16_kernel<D, true, D == 64, true>, 512, 0);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attn_fwd_bf16_kernel<D, true, false, true>, 512, 0);
  return e == hipSuccess ? n : 0;
}
template int fwd_bf16_wgs_per_cu<64>(bool);
template int fwd_bf16_wgs_per_cu<128>(bool);

template hipError_t launch_attn_bf16<64, true>(const FwdParams &, const RopeTable &, hipStream_t,
                                                    hipEvent_t, hipEvent_t);
template hipError_t launch_attn_bf16<64, false>(const FwdParams &, const RopeTable &, hipStream_t,
                                                    hipEvent_t, hipEvent_t);
template hipError_t launch_attn_bf16<128, true>(const FwdParams &, const RopeTable &, hipStream_t,
                                                    hipEvent_t, hipEvent_t);
template hipError_t launch_attn_bf16<128, false>(const FwdParams &, const RopeTable &, hipStream_t,
                                                    hipEvent_t, hipEvent_t);

}  // namespace attn
