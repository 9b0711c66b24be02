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
// work to overlap with the exponentials: the two 32-key score blocks run as two interleaved
// MFMA chains, then the P.V product of the previous tile carries the exponentials of both.
// The probabilities of a tile wait in registers, packed to bf16, until the next step.
//
// Softmax without a per-block maximum.  The running maximum m only needs to keep 2^(s - m)
// finite: interior tiles take probabilities against m as it stands (the QK accumulation starts
// from -m, so the products come out already shifted), and a tile is re-done with an exact
// maximum (scores recomputed from the still-staged K tile, accumulator and sum rescaled) only if
// its probability sum exceeds 2^64.  The first tile of a row block, tiles on the diagonal and
// the tile at the sequence end always take the exact maximum.  bf16 and fp32 hold values up to
// 2^64 with the same relative precision as values below 1, and out = o / l,
// lse = m + log2 l do not depend on which m was used.  The row sum adds the bf16-rounded
// probabilities (the values the P.V product sees) with a two-term dot product.

#include <hip/hip_ext.h>

#include "attn_device.h"

#define LDS_AS __attribute__((address_space(3)))

namespace attn {

constexpr int BN = 64;                      // keys per staged tile
constexpr float kSumLimit = 1.8446744e19f;  // 2^64: above this a tile is redone exactly
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// Raw (unformatted, byte-addressed) buffer resource over `bytes` bytes at `base`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int kReadsAhead = 4;  // LDS operand reads kept in flight ahead of the MFMAs

template <int D, bool CAUSAL>
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
  // rotation frequencies, read per row block from LDS rather than held in registers
  __shared__ double freq[D / 2];

  const int tid = threadIdx.x;
  if (tid < D / 2) freq[tid] = tab.rev[tid];
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep in SGPRs
  const int grp = wave >> 2;
  const int gw = wave & 3;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work: unit (b, g, head group) and row-block pair
  const int HG = p.G / p.hpw;
  const int u = blockIdx.x % p.n_units;
  const int pi = blockIdx.x / p.n_units;
  const int hg = u % HG;
  const int bg = u / HG;
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;
  const int S = p.S;
  const int RPB = p.rows_per_blk;
  const int r_lo = pi;
  const int r_hi = p.n_row_blocks - 1 - pi;
  const int t_lo = ((CAUSAL ? min(S, (r_lo + 1) * RPB) : S) + BN - 1) / BN;
  const int t_hi = ((CAUSAL ? min(S, (r_hi + 1) * RPB) : S) + BN - 1) / BN;
  const bool two = r_lo != r_hi;
  const int x = two ? (t_hi - t_lo) / 2 : t_hi / 2;  // key tiles of block r_hi run by group A
  // group A: segment 0 = (r_lo, tiles [0, t_lo)) when two, then segment 1 = (r_hi, [0, x));
  // group B: segment 1 = (r_hi, [x, t_hi)).
  const int len0 = (grp == 0 && two) ? t_lo : 0;
  const int k1s = grp == 0 ? 0 : x;
  const int n_mine = len0 + (grp == 0 ? x : t_hi - x);
  // group A issues the tile copies of both groups (it finishes its tiles first and would
  // otherwise wait at the barrier); group B's tile list is x, x+1, ..., t_hi-1
  const int len0_a = two ? t_lo : 0;
  const int n_a = len0_a + x;
  const int n_b = t_hi - x;
  // one extra step drains the last tile's P.V product; rounded up to even (the loop body is
  // two steps, and steps past a group's last tile only wait at the barrier)
  const int n_iter = (max((two ? t_lo : 0) + x, t_hi - x) + 2) & ~1;

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

  auto tile_of = [&](int i) { return i < len0 ? i : k1s + (i - len0); };
  auto tile_a = [&](int i) { return i < len0_a ? i : i - len0_a; };
  // this wave's share (DMA_PER_WAVE KiB) of copying tile kt of `buf` to dst
  auto stage = [&](__amdgpu_buffer_rsrc_t buf, int kt, char *dst) {
#pragma unroll
    for (int r = 0; r < DMA_PER_WAVE; ++r) {
      const int blk = gw * DMA_PER_WAVE + r;
      lds_dma16(buf, dma_lane, (uint32_t)kt * TB + blk * 1024, dst + blk * 1024);
    }
  };

  // ---- state of this wave's 32 rows
  bf16x8 qf[NKK];
  float m_run = -INFINITY;  // running maximum used for the probabilities (base-2 scores)
  float l_run = 0.f;        // this lane half's share of the running row sum
  f32x16 o[NCB];
  bf16x8 pend[2][2];        // probabilities of the previous tile, [block][key half]; zero if none
  int row0 = 0, kb_last = -1, cur_seg = -1;
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int t = 0; t < 2; ++t) pend[jb][t] = bf16x8{};
  // The P.V product of a step always runs; with zero probabilities it must read finite values,
  // so the V^T buffers start out zeroed (later they only ever hold staged tiles).
  {
    u32x4 *z0 = reinterpret_cast<u32x4 *>(ldsv0);
    u32x4 *z1 = reinterpret_cast<u32x4 *>(ldsv1);
#pragma unroll
    for (int r = 0; r < 2 * TB / 16 / 512; ++r) {
      z0[tid + 512 * r] = u32x4{0u, 0u, 0u, 0u};
      z1[tid + 512 * r] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  auto begin_seg = [&](int seg) {
    const int R = seg == 0 ? r_lo : r_hi;
    row0 = R * RPB + sub * 32;
    kb_last = row0 >= S ? -1 : (CAUSAL ? min(row0 + 31, S - 1) : S - 1) / 32;
    const int my_row = row0 + l32;
    u32x4 raw[NKK];
    if (my_row < S) {
      const __bf16 *src = p.q + (((size_t)b * S + my_row) * p.Hq + head) * D + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) raw[kk] = *reinterpret_cast<const u32x4 *>(src + 16 * kk);
    } else {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) raw[kk] = u32x4{0u, 0u, 0u, 0u};
    }
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
          const float t = turn_fraction(my_row, f);
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
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{};
  };

  auto store_seg = [&]() {
    const float l_tot = l_run + xor32(l_run);
    const int my_row = row0 + l32;
    if (my_row < S) {
      const float inv = 1.0f / l_tot;
      __bf16 *dst = p.out + (((size_t)b * S + my_row) * p.Hq + head) * D + 4 * hh;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          u32x2 w2;
          w2[0] = pack_bf16x2(o[cb][4 * a + 0] * inv, o[cb][4 * a + 1] * inv);
          w2[1] = pack_bf16x2(o[cb][4 * a + 2] * inv, o[cb][4 * a + 3] * inv);
          *reinterpret_cast<u32x2 *>(dst + 32 * cb + 8 * a) = w2;
        }
      if (hh == 0)
        p.lse[((size_t)b * p.Hq + head) * S + my_row] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
    }
  };

  // ---- block pieces (kd / vd: this group's K and V^T tile)
  auto kfrag = [&](const char *kd, int jb, int kk) {
    return *reinterpret_cast<const bf16x8 *>(kd + k_lane + 2 * kk * 1024 + jb * 512);
  };
  auto vfrag = [&](const char *vd, int jb, int t, int cb) {
    return *reinterpret_cast<const bf16x8 *>(vd + v_lane + (4 * jb + 2 * t) * 16 * D + cb * 512);
  };
  auto qk = [&](const char *kd, int jb) {
    f32x16 sc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) sc = mfma(kfrag(kd, jb, kk), qf[kk], sc);
    return sc;
  };
  // O += V^T(previous tile) P^T(previous tile)
  auto pv_pending = [&](const char *vd) {
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o[cb] = mfma(vfrag(vd, jb, t, cb), pend[jb][t], o[cb]);
  };
  // keys after the query or past the sequence end get -inf (only called where some may be)
  auto mask = [&](f32x16 &sc, int kb0) {
    const int my_row = row0 + l32;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = kb0 + 8 * (v >> 2) + 4 * hh + (v & 3);
      if ((CAUSAL && j > my_row) || j >= S) sc[v] = -INFINITY;
    }
  };
  // p = 2^(sc - m) packed to bf16; returns this lane's sum of the bf16-rounded probabilities
  auto expo_pack = [&](f32x16 &sc, float m, bf16x8 (&pb)[2]) {
#pragma unroll
    for (int v = 0; v < 16; ++v) sc[v] = __builtin_amdgcn_exp2f(sc[v] - m);
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 pw;
#pragma unroll
      for (int w = 0; w < 4; ++w) pw[w] = pack_bf16x2(sc[8 * t + 2 * w], sc[8 * t + 2 * w + 1]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // through a scalar: a bit cast of the vector element itself reads element 0
        const uint32_t pair = pw[w];
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                             __builtin_bit_cast(bf16x2, kOnesBf16x2), rs, false);
      }
      pb[t] = __builtin_bit_cast(bf16x8, pw);
    }
    return rs;
  };
  auto needs_redo = [&](float rsum) {
    return __builtin_amdgcn_ballot_w64(!(rsum <= kSumLimit)) != 0;  // also catches inf and NaN
  };

  // one probability pair: p = 2^(s - m) for elements 2w2, 2w2 + 1, packed to bf16 into
  // pw[w2 / 4][w2 % 4], the bf16 values added to the row sum rs
  auto exp_pair = [&](const f32x16 &sc, int w2, float m, u32x4 (&pw)[2], float &rs) {
    const float e0 = __builtin_amdgcn_exp2f(sc[2 * w2] - m);
    const float e1 = __builtin_amdgcn_exp2f(sc[2 * w2 + 1] - m);
    const uint32_t pk = pack_bf16x2(e0, e1);
    rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), __builtin_bit_cast(bf16x2, kOnesBf16x2),
                                         rs, false);
    // consumed here, so the pair is computed in the unit that asks for it (the copy branches
    // of group A would otherwise let the compiler sink it to the end of the phase)
    asm volatile("" ::"v"(rs));
    pw[w2 >> 2][w2 & 3] = pk;
  };

  // One key tile: QK(b0) and QK(b1) as two interleaved chains | PV(previous tile) with
  // exp(b0), exp(b1), the probabilities taken against the running m.  The issue order is written out: each unit is
  // one MFMA, the operand read kReadsAhead MFMAs ahead and a share of the exponentials, fenced
  // so the compiler keeps it.  If any row's sum passed the limit, or m was not yet set (the
  // first tile of a row block gives inf / NaN sums), the tile is redone with the exact maximum
  // over both blocks: scores recomputed from the still-staged K tile, the state rescaled to the
  // new maximum, probabilities recomputed.
  constexpr int NPV = 4 * NCB;               // MFMAs of the P.V product of one tile
  constexpr int NMF = 2 * NKK + NPV;         // MFMAs of one tile
  constexpr int NDMA = 4 * DMA_PER_WAVE;     // copy instructions per step of a group-A wave
  auto pv_of = [&](const char *vd, int r) {  // operand of the r-th P.V MFMA
    const int jb = r / (2 * NCB), t = (r / NCB) % 2, cb = r % NCB;
    return vfrag(vd, jb, t, cb);
  };
  // The four tile copies of a step (next K tile and this V^T tile, of each group) as source /
  // destination pairs; a group-A wave moves its share of each, one instruction every
  // NMF / NDMA MFMAs, so the copies pass through the vector memory path while the tile's
  // arithmetic runs instead of stalling every wave at the start of a step.
  struct Copies {
    int tile[4];  // K tile, V^T tile, K tile, V^T tile
    char *dst[4];
  };
  auto copy_part = [&](const Copies &c, int r) {
    const int q = r / DMA_PER_WAVE;
    const int blk = gw * DMA_PER_WAVE + r % DMA_PER_WAVE;
    lds_dma16((q & 1) ? vt_buf : kr_buf, dma_lane, (uint32_t)c.tile[q] * TB + blk * 1024, c.dst[q] + blk * 1024);
  };
  auto tile = [&](const char *kd, const char *vd, int kb0, bool msk, const Copies &cp) {
    auto dma_at = [&](int g) {  // after the g-th MFMA of the tile (group A only)
      if ((g * NDMA) % NMF == 0 && grp == 0) copy_part(cp, g * NDMA / NMF);
    };
    // operand reads: phase 1 reads K fragments in MFMA order (k0, k1 alternating blocks), the
    // last ones of phase 1 fetch the first P.V operands
    auto k_of = [&](int g) { return kfrag(kd, g & 1, g >> 1); };
    bf16x8 fr[kReadsAhead];
#pragma unroll
    for (int r = 0; r < kReadsAhead; ++r) fr[r] = k_of(r);
    // phase 1: QK(b0) and QK(b1) as two interleaved accumulation chains
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int g = 0; g < 2 * NKK; ++g) {
      if (g & 1)
        s1 = mfma(fr[g % kReadsAhead], qf[g >> 1], s1);
      else
        s0 = mfma(fr[g % kReadsAhead], qf[g >> 1], s0);
      const int nx = g + kReadsAhead;
      fr[g % kReadsAhead] = nx < 2 * NKK ? k_of(nx) : pv_of(vd, nx - 2 * NKK);
      dma_at(g);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (msk) {
      mask(s0, kb0);
      mask(s1, kb0 + 32);
    }
    __builtin_amdgcn_sched_barrier(0);
    // phase 2: PV(previous tile) with exp(b0) and exp(b1)
    u32x4 pw0[2], pw1[2];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int r = 0; r < NPV; ++r) {
      const int jb = r / (2 * NCB), t = (r / NCB) % 2, cb = r % NCB;
      o[cb] = mfma(fr[r % kReadsAhead], pend[jb][t], o[cb]);
      if (r + kReadsAhead < NPV) fr[r % kReadsAhead] = pv_of(vd, r + kReadsAhead);
      dma_at(2 * NKK + r);
#pragma unroll
      for (int w2 = r * 16 / NPV; w2 < (r + 1) * 16 / NPV; ++w2) {
        if (w2 < 8)
          exp_pair(s0, w2, m_run, pw0, rs0);
        else
          exp_pair(s1, w2 - 8, m_run, pw1, rs1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 p0[2], p1[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      p0[t] = __builtin_bit_cast(bf16x8, pw0[t]);
      p1[t] = __builtin_bit_cast(bf16x8, pw1[t]);
    }
    if (__builtin_expect(needs_redo(rs0 + rs1), 0)) {
      asm volatile("" ::: "memory");  // re-read the K fragments from LDS
      s0 = qk(kd, 0);
      s1 = qk(kd, 1);
      if (msk) {
        mask(s0, kb0);
        mask(s1, kb0 + 32);
      }
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, fmaxf(s0[v], s1[v]));
      const float m_new = fmaxf(m_run, max_xor32(mx));
      // a row with no visible key so far keeps m = -inf and gets zero probabilities
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);  // 0 when m was unset
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
      m_run = m_new;
      rs0 = expo_pack(s0, m_use, p0);
      rs1 = expo_pack(s1, m_use, p1);
    }
    l_run += rs0 + rs1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      pend[0][t] = p0[t];
      pend[1][t] = p1[t];
    }
  };

  // ---- main loop.  Step i: K tile i in ldsk[i%2], V^T tile i-1 in ldsv[(i+1)%2]; copies of
  // K tile i+1 into ldsk[(i+1)%2] and V^T tile i into ldsv[i%2], issued by the tile, run
  // meanwhile.  Unrolled by
  // two so the buffer of every access is known at compile time.  Step n_mine only finishes
  // the last tile's P.V product; steps after it only wait.
  auto step = [&](int i, const char *kcur, char *knxt, const char *vprev, char *vfill) {
    const int go = grp * TB;
    const int seg = i < n_mine ? (i < len0 ? 0 : 1) : -1;
    if (seg != cur_seg) {  // new row block, or the end of this group's tiles
      if (cur_seg >= 0) {
        pv_pending(vprev + go);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int t = 0; t < 2; ++t) pend[jb][t] = bf16x8{};
        if (cur_seg == 0) store_seg();  // the r_hi block is stored (or merged) after the loop
      }
      if (seg >= 0) begin_seg(seg);
      cur_seg = seg;
    }
    // copies of this step: K tile i+1 and V^T tile i of each group.  Indices past a group's
    // last tile are clamped to it: the copy is then an in-bounds duplicate into a buffer that
    // group no longer reads.
    Copies cp;
    {
      const int ia = max(min(i, n_a - 1), 0), ia1 = max(min(i + 1, n_a - 1), 0);
      const int ib = min(i, n_b - 1), ib1 = min(i + 1, n_b - 1);
      cp.tile[0] = tile_a(ia1);
      cp.dst[0] = knxt;
      cp.tile[1] = tile_a(ia);
      cp.dst[1] = vfill;
      cp.tile[2] = x + ib1;
      cp.dst[2] = knxt + TB;
      cp.tile[3] = x + ib;
      cp.dst[3] = vfill + TB;
    }
    if (seg >= 0) {
      const int kt = tile_of(i);
      const int kb0 = kt * BN;
      const bool msk = (CAUSAL && kb0 + BN - 1 > row0) || kb0 + BN > S;
      tile(kcur + go, vprev + go, kb0, msk, cp);
    } else if (grp == 0 && i < n_b) {  // group A is done but B still needs its tiles
#pragma unroll
      for (int r = 0; r < NDMA; ++r) copy_part(cp, r);
    }
    wait_vm_all();
    __syncthreads();
  };
  if (grp == 0) {  // first K tiles of both groups
    stage(kr_buf, 0, ldsk0);
    stage(kr_buf, x, ldsk0 + TB);
  }
  wait_vm_all();
  __syncthreads();
  for (int i = 0; i < n_iter; i += 2) {
    step(i, ldsk0, ldsk1, ldsv1, ldsv0);
    step(i + 1, ldsk1, ldsk0, ldsv0, ldsv1);
  }

  // ---- finish: the split block r_hi is merged in B.  The tile buffers are free after the last
  // barrier: per-wave accumulators of group A go to ldsk0 (waves 0, 1) and ldsk1 (waves 2, 3),
  // maxima and sums to ldsv0.
  if (x > 0) {
    float *mo = reinterpret_cast<float *>(gw < 2 ? ldsk0 : ldsk1) + (gw & 1) * NCB * 16 * 64;
    float *mm = reinterpret_cast<float *>(ldsv0);
    if (grp == 0) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mo[(cb * 16 + v) * 64 + lane] = o[cb][v];
      mm[gw * 64 + lane] = m_run;
      mm[256 + gw * 64 + lane] = l_run;
    }
    __syncthreads();
    if (grp == 1) {
      const float ma = mm[gw * 64 + lane];
      const float la = mm[256 + gw * 64 + lane];
      const float m_new = fmaxf(ma, m_run);  // finite for every row below S
      const float ca = __builtin_amdgcn_exp2f(ma - m_new);
      const float cb_ = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run = la * ca + l_run * cb_;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[cb][v] = mo[(cb * 16 + v) * 64 + lane] * ca + o[cb][v] * cb_;
      m_run = m_new;
    }
  }
  if (grp == 1) store_seg();
}

template <int D, bool CAUSAL>
hipError_t launch_attn_bf16(const FwdParams &p, const RopeTable &tab, hipStream_t stream,
                            hipEvent_t ev_start, hipEvent_t ev_stop) {
  const long long blocks = (long long)p.n_units * p.n_pairs;
  hipExtLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(512), 0, stream,
                        ev_start, ev_stop, 0, p, tab);
  return hipGetLastError();
}

template hipError_t launch_attn_bf16<64, true>(const FwdParams &, const RopeTable &, hipStream_t,
                                                    hipEvent_t, hipEvent_t);
template hipError_t launch_attn_bf16<64, false>(const FwdParams &, const RopeTable &, hipStream_t,
                                                    hipEvent_t, hipEvent_t);
template hipError_t launch_attn_bf16<128, true>(const FwdParams &, const RopeTable &, hipStream_t,
                                                    hipEvent_t, hipEvent_t);
template hipError_t launch_attn_bf16<128, false>(const FwdParams &, const RopeTable &, hipStream_t,
                                                    hipEvent_t, hipEvent_t);

}  // namespace attn
