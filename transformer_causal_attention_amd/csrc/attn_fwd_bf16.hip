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
// into LDS (global_load_lds, 16 bytes per lane, no registers) as one contiguous run, double
// buffered per group, and every MFMA operand is then one 16-byte LDS read at a per-lane base
// plus a constant offset, with 8 consecutive lanes reading 128 consecutive bytes (no bank
// conflicts, no address arithmetic in the loop).  The two buffers are separate LDS arrays and
// the loop is unrolled by two, so the compiler can see that operand reads of one buffer never
// depend on the copies filling the other and inserts no wait for them.
//
// Matrix layout.  With A = K tile (32 keys x 16 dims) and B = Q^T (16 dims x 32 rows), the
// 32x32x16 bf16 MFMA yields S^T: lane l holds query row l%32 and, in its 16 accumulators,
// keys 8*(v/4) + 4*(l/32) + v%4.  Row sums are thus in-lane plus one exchange between the lane
// halves at the end.  O^T = V^T P^T takes those accumulators (packed to bf16) as its B operand
// unchanged; the matching A operand (V^T, 8 keys of one column in that order) is one 16-byte
// read, because V^T stores each group of 16 keys in exactly that order.  Keys above the
// diagonal are never loaded, and a wave skips the 32-key blocks entirely above its rows.
//
// Softmax without a per-block maximum.  The running maximum m only needs to keep 2^(s - m)
// finite: probabilities are taken against m as it stands, and a block is re-done with an
// exact maximum (K fragments re-read, scores recomputed, accumulator and sum rescaled) only
// if its probability sum exceeds 2^64.  The first block of a row block sets m exactly.  bf16
// and fp32 hold values up to 2^64 with the same relative precision as values below 1, and the
// result out = o / l, lse = m + log2 l does not depend on which m was used.  The common path
// is branch-free, so a tile runs as  QK(b0) | QK(b1) with exp(b0) | PV(b0) with exp(b1) |
// PV(b1), letting the in-order wave issue the exponentials of one block between the MFMAs of
// the other.

#include <type_traits>

#include <hip/hip_ext.h>

#include "attn_device.h"

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

namespace attn {

constexpr int BN = 64;                      // keys per staged tile
constexpr float kSumLimit = 1.8446744e19f;  // 2^64: above this a block is redone exactly

__device__ __forceinline__ float xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0] holds lane l%32's value in every lane, r[1] lane 32 + l%32's
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Each lane copies 16 bytes from `g` to lds_base + 16 * lane (lds_base is wave-uniform).
__device__ __forceinline__ void lds_dma16(const void *g, char *lds_base) {
  __builtin_amdgcn_global_load_lds((GLB_AS void *)g, (LDS_AS void *)lds_base, 16, 0, 0);
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512) attn_fwd_bf16_kernel(FwdParams p, RopeTable tab) {
  constexpr int NKK = D / 16;              // MFMA steps over head_dim
  constexpr int NCB = D / 32;              // 32-column blocks of the output
  constexpr int TB = BN * D * 2;           // bytes of one staged K or V^T tile
  constexpr int DMA_PER_WAVE = TB / 4096;  // 1 KiB copies per wave, tile and operand
  // one array per buffer parity, each [group][K, V^T]
  __shared__ __attribute__((aligned(1024))) char lds0[4 * TB];
  __shared__ __attribute__((aligned(1024))) char lds1[4 * TB];
  // rotation frequencies, read per row block from LDS rather than held in registers (kept as
  // loop-invariant values they would occupy 2*D VGPRs for the whole loop)
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
  const int n_iter = max((two ? t_lo : 0) + x, t_hi - x);

  const int head = g * p.G + hg * p.hpw + (gw % p.hpw);
  const int sub = gw / p.hpw;

  const size_t n_tiles = (size_t)(p.S_pad / BN);
  const char *kr_tiles = reinterpret_cast<const char *>(p.kr) + ((size_t)b * p.Hkv + g) * n_tiles * TB;
  const char *vt_tiles = reinterpret_cast<const char *>(p.vt) + ((size_t)b * p.Hkv + g) * n_tiles * TB;

  // per-lane operand bases inside a staged tile (constant parts are immediates):
  //   K of key block jb, step kk:   [chunk 2kk + hh][key 32jb + l32] -> k_lane + 2kk*1024 + jb*512
  //   V^T of block jb, half t, cb:  [chunk 4jb + 2t + hh][column 32cb + l32]
  //                                 -> v_lane + (4jb + 2t)*16*D + cb*512
  const int k_lane = hh * 1024 + l32 * 16;
  const int v_lane = hh * 16 * D + l32 * 16;

  auto stage = [&](int i, char *dst) {
    const int kt = i < len0 ? i : k1s + (i - len0);
    char *kd = dst + grp * 2 * TB;
    const char *ks = kr_tiles + (size_t)kt * TB;
    const char *vs = vt_tiles + (size_t)kt * TB;
#pragma unroll
    for (int r = 0; r < DMA_PER_WAVE; ++r) {
      const int blk = gw * DMA_PER_WAVE + r;
      lds_dma16(ks + blk * 1024 + lane * 16, kd + blk * 1024);
      lds_dma16(vs + blk * 1024 + lane * 16, kd + TB + blk * 1024);
    }
  };

  // ---- state of this wave's 32 rows
  bf16x8 qf[NKK];
  float m_run = -INFINITY;  // running maximum used for the probabilities (base-2 scores)
  float l_run = 0.f;        // this lane half's share of the running row sum
  f32x16 o[NCB];
  int row0 = 0, kb_last = -1, cur_seg = -1;

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

  // ---- block pieces (kd / vd: this group's K and V^T tile in the current buffer)
  auto qk = [&](const char *kd, int jb) {
    bf16x8 kf[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kf[kk] = *reinterpret_cast<const bf16x8 *>(kd + k_lane + 2 * kk * 1024 + jb * 512);
    f32x16 sc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) sc = mfma(kf[kk], qf[kk], sc);
    return sc;
  };
  auto load_v = [&](const char *vd, int jb, bf16x8 (&vf)[2][NCB]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        vf[t][cb] = *reinterpret_cast<const bf16x8 *>(vd + v_lane + (4 * jb + 2 * t) * 16 * D + cb * 512);
  };
  // keys after the query (diagonal block) or past the sequence end get -inf
  auto mask = [&](f32x16 &sc, int kb0) {
    if ((CAUSAL && kb0 + 31 > row0) || kb0 + 32 > S) {  // wave-uniform
      const int my_row = row0 + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = kb0 + 8 * (v >> 2) + 4 * hh + (v & 3);
        if ((CAUSAL && j > my_row) || j >= S) sc[v] = -INFINITY;
      }
    }
  };
  // exact maximum of a (masked) block; rescales the accumulated state to it.  Finite: every
  // row of a processed block has a visible key.
  auto take_max = [&](const f32x16 &sc) {
    float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
    for (int v = 2; v < 16; ++v) mx = fmaxf(mx, sc[v]);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run was unset
    l_run *= alpha;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
    m_run = m_new;
  };
  // p = 2^(s - m_run) in place; returns this lane's sum of the block
  auto expo = [&](f32x16 &sc) {
    float rsum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      sc[v] = __builtin_amdgcn_exp2f(sc[v] - m_run);
      rsum += sc[v];
    }
    return rsum;
  };
  auto needs_redo = [&](float rsum) {
    return __builtin_amdgcn_ballot_w64(!(rsum <= kSumLimit)) != 0;  // also catches inf and NaN
  };
  // exact path for a block whose probability sum overflowed the limit: scores recomputed from
  // the (still staged) K tile, maximum taken, state rescaled, probabilities recomputed
  auto redo = [&](f32x16 &sc, float &rsum, const char *kd, int jb, int kb0) {
    // re-read the fragments rather than keeping the first read's registers alive until here
    asm volatile("" ::: "memory");
    sc = qk(kd, jb);
    mask(sc, kb0);
    take_max(sc);
    rsum = expo(sc);
  };
  auto pv = [&](const f32x16 &pr, const bf16x8 (&vf)[2][NCB]) {
    bf16x8 pb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 pw;
#pragma unroll
      for (int w = 0; w < 4; ++w) pw[w] = pack_bf16x2(pr[8 * t + 2 * w], pr[8 * t + 2 * w + 1]);
      pb[t] = __builtin_bit_cast(bf16x8, pw);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) o[cb] = mfma(vf[t][cb], pb[t], o[cb]);
  };

  auto compute_tile = [&](int kt, const char *base) {
    const char *kd = base + grp * 2 * TB;
    const char *vd = kd + TB;
    const int kb0 = kt * BN;
    if (2 * kt > kb_last) return;  // the whole tile is above this wave's rows
    f32x16 s0 = qk(kd, 0);
    mask(s0, kb0);
    if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY)) take_max(s0);  // first block of the rows
    if (2 * kt + 1 <= kb_last) {
      // QK(b1) with exp(b0) | PV(b0) with exp(b1) | PV(b1); the fences keep each region's
      // fragment loads inside it, which bounds the live registers
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s1 = qk(kd, 1);
      float r0 = expo(s0);
      __builtin_amdgcn_sched_barrier(0);
      if (needs_redo(r0)) redo(s0, r0, kd, 0, kb0);
      l_run += r0;
      mask(s1, kb0 + 32);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 vf[2][NCB];
      load_v(vd, 0, vf);
      pv(s0, vf);
      float r1 = expo(s1);
      __builtin_amdgcn_sched_barrier(0);
      if (needs_redo(r1)) redo(s1, r1, kd, 1, kb0 + 32);
      l_run += r1;
      __builtin_amdgcn_sched_barrier(0);
      load_v(vd, 1, vf);
      pv(s1, vf);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      float r0 = expo(s0);
      if (needs_redo(r0)) redo(s0, r0, kd, 0, kb0);
      l_run += r0;
      bf16x8 vf[2][NCB];
      load_v(vd, 0, vf);
      pv(s0, vf);
    }
  };

  // ---- main loop: both groups step through their tile lists in lockstep; tile i sits in
  // buffer i % 2 (unrolled by two so the buffer of every access is known at compile time)
  auto step = [&](int i, const char *cur, char *nxt) {
    if (i + 1 < n_mine) stage(i + 1, nxt);
    if (i < n_mine) {
      const int seg = i < len0 ? 0 : 1;
      if (seg != cur_seg) {
        if (cur_seg == 0) store_seg();
        begin_seg(seg);
        cur_seg = seg;
      }
      compute_tile(i < len0 ? i : k1s + (i - len0), cur);
    }
    wait_vm_all();
    __syncthreads();
  };
  if (n_mine > 0) stage(0, lds0);
  wait_vm_all();
  __syncthreads();
  for (int i = 0; i < n_iter; i += 2) {
    step(i, lds0, lds1);
    if (i + 1 < n_iter) step(i + 1, lds1, lds0);
  }

  // ---- finish: A stores block r_lo if it still holds it; the split block is merged in B
  if (grp == 0 && cur_seg == 0) store_seg();
  if (x > 0) {
    float *mo = reinterpret_cast<float *>(lds0);  // tile buffers are free after the last barrier
    float *mm = reinterpret_cast<float *>(lds1);
    if (grp == 0) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mo[((gw * NCB + cb) * 16 + v) * 64 + lane] = o[cb][v];
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
        for (int v = 0; v < 16; ++v) o[cb][v] = mo[((gw * NCB + cb) * 16 + v) * 64 + lane] * ca + o[cb][v] * cb_;
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
