// Backward pass of the fused causal RoPE-GQA attention for gfx950: dq, dk, dv from q, k, v,
// the forward's out and lse, and the output gradient dout.
//
// The gradient of the forward (Picotron, PaLM and llama3-from-scratch pages define the
// forward; the PaLM page's wrapper trains it with a cross-entropy loss, section 2.7):
//   P = exp(s - lse) with s = q'.k'/sqrt(D) (q', k' rotated), recomputed from the saved lse;
//   dv_g = sum over the group's heads of P^T dout;   dP = dout v^T;
//   ds = P (dP - rowsum(dout * out));
//   dq' = ds k' / sqrt(D);   dk'_g = sum over the group's heads of ds^T q' / sqrt(D);
//   dq = R^T dq', dk = R^T dk' (the rotation by minus the position's angles).
//
// 32-row blocks of queries and keys throughout.  Kernels (head_dim 64 and 128 here; the
// head_dim 256 ones, which keep their fixed block in LDS, are in attn_bwd_d256.hip):
//   bwd_prep            the layout passes, one launch: per query block rotated queries (scaled)
//                       in "c" and "t" layouts, dout in both, and per row lse * log2(e) and
//                       rowsum(dout * out); per key block rotated keys in "c" and "t" layouts
//                       and values in "c" layout;
//   dk, dv              bwd_dkdv_shared_item: a workgroup of four waves takes four consecutive
//                       key blocks of one K/V head (one each) and the query heads of its head
//                       split; each query block's tiles are copied once into LDS, where every
//                       wave reads its operands: S = Q K^T (and dP = dO V^T) with one key per
//                       lane, then dv += P^T dO or dk += dS^T Q (both in one pass at head_dim
//                       64), summed over the heads in registers; dk is rotated back and each row
//                       written once (no atomics), or, with head splits, left as fp32 partials
//                       for bwd_part_reduce;
//   dq                  bwd_dq_shared_item (a workgroup of four waves: up to four query heads
//                       of a K/V group times consecutive query blocks, each key block's tiles
//                       copied once into LDS): S^T = K Q^T and dP^T = V dO^T with one query
//                       per lane, dq += dS K, rotated back and written;
//   bwd_dkdv_shared_kernel  runs the dk, dv and (four heads per workgroup) dq work items in one
//                       launch, heaviest first, when they fit on the GPU at once, else dk and dv
//                       items in launches of their own;
//   bwd_part_reduce     adds the head splits' partials in split order;
//   bwd_dkdv, bwd_dq    per-wave kernels with operands from L2 (one wave per query head and
//                       block or block pair), kept as diagnostics (ATTN_BWD_KV, ATTN_BWD_DQ) and
//                       checked against the shared ones.
// A call may be one block of a longer sequence (one step of ring attention's backward): queries
// at positions q_pos0 + i, keys at k_pos0 + j, key j visible to query i iff j <= i + delta with
// delta = q_pos0 - k_pos0; out and lse are then the forward's results over every key block, and
// dq (dk, dv) is this key block's (query block's) part of the gradient.  Block kb of keys is seen
// by query blocks from qb_lo(kb) on, query block qb sees key blocks below kb_end(qb), and a
// block needs the element mask only where some key is later than some row.  Every MFMA operand
// is one 16-byte read per lane from the pre-laid-out tiles, in LDS or (per-wave kernels) in
// registers, each register reloaded with the next block's operand as soon as its instruction
// has read it.
//
// MFMA v_mfma_f32_32x32x16_bf16: A lane l holds row l%32, k = 8(l/32) .. +7; B lane l holds
// column l%32, same k; the result's register v in lane l is row 8(v/4) + 4(l/32) + v%4,
// column l%32.  A score result packed as bf16 (registers 8t .. 8t+7 -> one operand) therefore
// lists its rows in the order 16t + swap23(8(l/32) + e), which is the row order of the "t"
// layout.

#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "attn_bwd_common.h"

namespace attn {

// ---------------------------------------------------------------------------------------------
// threads of a layout-pass workgroup: one per item (32 rows x D/16 chunk pairs), at most 256
template <int D>
constexpr int bwd_prep_threads() {
  return BR * (D / 16) < 256 ? BR * (D / 16) : 256;
}

// Layout passes.  bwd_prep_threads<D>() threads, one per item (two items each at head_dim 256);
// item = row * NCH + c covers dims 8c .. 8c+7 and D/2 + 8c .. of one row (NCH = D/16 pairs of
// 8-dim chunks).

// key block blk of (b, K/V head) blk / NB, staged through sk (32 rows of D + 8)
template <int D>
__device__ __forceinline__ void bwd_prep_k_item(const BwdParams &p, const RopeTable &tab, int blk, uint16_t *sk) {
  constexpr int NCH = D / 16;
  constexpr int LS = D + 8;
  constexpr int T = BR * D;  // elements per tile
  const int tid = threadIdx.x;
  const int kb = blk % p.NB;
  const int unit = blk / p.NB;  // b * Hkv + g
  const int g = unit % p.Hkv, b = unit / p.Hkv;
  const size_t tile = (size_t)blk * T;
  for (int item = tid; item < BR * NCH; item += bwd_prep_threads<D>()) {  // one pass, two at head_dim 256
    const int row = item / NCH, c = item % NCH;
    const int r = kb * BR + row;
    u32x4 kx = {0u, 0u, 0u, 0u}, ky = kx, vx = kx, vy = kx;
    if (r < p.S) {
      const size_t src = (((size_t)b * p.S + r) * p.Hkv + g) * D + 8 * c;
      if (tab.interleaved) {  // adjacent-pair form: dims 16c .. 16c+15 as evens and odds
        const size_t ks = src + 8 * c;
        deinterleave16(*reinterpret_cast<const u32x4 *>(p.k + ks), *reinterpret_cast<const u32x4 *>(p.k + ks + 8), kx, ky);
      } else {
        kx = *reinterpret_cast<const u32x4 *>(p.k + src);
        ky = *reinterpret_cast<const u32x4 *>(p.k + src + D / 2);
      }
      vx = *reinterpret_cast<const u32x4 *>(p.v + src);
      vy = *reinterpret_cast<const u32x4 *>(p.v + src + D / 2);
    }
    float x[8], y[8];
    rotate8<D>(tab, c, p.k_pos0 + r, kx, ky, x, y);
    const u32x4 wx = r < p.S ? pack8(x, 1.f) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 wy = r < p.S ? pack8(y, 1.f) : u32x4{0u, 0u, 0u, 0u};
    // c layout: chunk c at [c][row][8]
    *reinterpret_cast<u32x4 *>(p.kc + tile + ((size_t)c * BR + row) * 8) = wx;
    *reinterpret_cast<u32x4 *>(p.kc + tile + ((size_t)(c + NCH) * BR + row) * 8) = wy;
    *reinterpret_cast<u32x4 *>(p.vc + tile + ((size_t)c * BR + row) * 8) = vx;
    *reinterpret_cast<u32x4 *>(p.vc + tile + ((size_t)(c + NCH) * BR + row) * 8) = vy;
    *reinterpret_cast<u32x4 *>(sk + row * LS + 8 * c) = wx;
    *reinterpret_cast<u32x4 *>(sk + row * LS + D / 2 + 8 * c) = wy;
  }
  __syncthreads();
  write_t_layout<D, LS>(sk, p.kt + tile, tid, bwd_prep_threads<D>());
}

// query block blk of (b, query head) blk / NB, staged through sq and sd
template <int D>
__device__ __forceinline__ void bwd_prep_q_item(const BwdParams &p, const RopeTable &tab, int blk, uint16_t *sq,
                                                uint16_t *sd) {
  constexpr int NCH = D / 16;
  constexpr int LS = D + 8;
  constexpr int T = BR * D;
  const int tid = threadIdx.x;
  const int qb = blk % p.NB;
  const int unit = blk / p.NB;  // b * Hq + h
  const int h = unit % p.Hq, b = unit / p.Hq;
  const size_t tile = (size_t)blk * T;
  // one pass, two at head_dim 256 (the NCH items of a row are consecutive lanes of one wave in
  // either pass, for the row sums below)
  for (int item = tid; item < BR * NCH; item += bwd_prep_threads<D>()) {
    const int row = item / NCH, c = item % NCH;
    const int r = qb * BR + row;
    const bool ok = r < p.S;
    u32x4 qx = {0u, 0u, 0u, 0u}, qy = qx, gx = qx, gy = qx, ox = qx, oy = qx;
    if (ok) {
      const size_t src = (((size_t)b * p.S + r) * p.Hq + h) * D + 8 * c;
      if (tab.interleaved) {  // adjacent-pair form: dims 16c .. 16c+15 as evens and odds
        const size_t qs = src + 8 * c;
        deinterleave16(*reinterpret_cast<const u32x4 *>(p.q + qs), *reinterpret_cast<const u32x4 *>(p.q + qs + 8), qx, qy);
      } else {
        qx = *reinterpret_cast<const u32x4 *>(p.q + src);
        qy = *reinterpret_cast<const u32x4 *>(p.q + src + D / 2);
      }
      gx = *reinterpret_cast<const u32x4 *>(p.dout + src);
      gy = *reinterpret_cast<const u32x4 *>(p.dout + src + D / 2);
      ox = *reinterpret_cast<const u32x4 *>(p.out + src);
      oy = *reinterpret_cast<const u32x4 *>(p.out + src + D / 2);
    }
    float x[8], y[8];
    rotate8<D>(tab, c, p.q_pos0 + r, qx, qy, x, y);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4 *>(p.qc + tile + ((size_t)c * BR + row) * 8) = ok ? pack8(x, p.scale_log2) : zero;
    *reinterpret_cast<u32x4 *>(p.qc + tile + ((size_t)(c + NCH) * BR + row) * 8) = ok ? pack8(y, p.scale_log2) : zero;
    *reinterpret_cast<u32x4 *>(sq + row * LS + 8 * c) = ok ? pack8(x, p.inv_sqrt_d) : zero;
    *reinterpret_cast<u32x4 *>(sq + row * LS + D / 2 + 8 * c) = ok ? pack8(y, p.inv_sqrt_d) : zero;
    *reinterpret_cast<u32x4 *>(p.dc + tile + ((size_t)c * BR + row) * 8) = gx;
    *reinterpret_cast<u32x4 *>(p.dc + tile + ((size_t)(c + NCH) * BR + row) * 8) = gy;
    *reinterpret_cast<u32x4 *>(sd + row * LS + 8 * c) = gx;
    *reinterpret_cast<u32x4 *>(sd + row * LS + D / 2 + 8 * c) = gy;
    // rowsum(dout * out) over this item's 16 dims, then over the NCH items of the row
    // (consecutive lanes of one wave)
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += bf16_lo(gx[i]) * bf16_lo(ox[i]) + bf16_hi(gx[i]) * bf16_hi(ox[i]);
      acc += bf16_lo(gy[i]) * bf16_lo(oy[i]) + bf16_hi(gy[i]) * bf16_hi(oy[i]);
    }
#pragma unroll
    for (int off = NCH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (c == 0) {
      const size_t ri = (size_t)unit * p.NB * BR + (size_t)qb * BR + row;
      p.dd[ri] = ok ? acc : 0.f;
      // a row with no visible key (lse -inf) has no gradient: +inf makes its weights 0 as for
      // rows past S
      const float lr = ok ? p.lse[((size_t)b * p.Hq + h) * p.S + r] : INFINITY;
      p.l2[ri] = lr == -INFINITY ? INFINITY : lr * 1.4426950408889634f;
    }
  }
  __syncthreads();
  write_t_layout<D, LS>(sq, p.qt + tile, tid, bwd_prep_threads<D>());
  write_t_layout<D, LS>(sd, p.dt + tile, tid, bwd_prep_threads<D>());
}

// Both layout passes in one launch: the B * Hq * NB query blocks (four tiles each), then the
// B * Hkv * NB key blocks.
template <int D>
__global__ void __launch_bounds__(bwd_prep_threads<D>()) bwd_prep_kernel(BwdParams p, RopeTable tab) {
  constexpr int LS = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t st[2 * BR * LS];
  const int qblocks = p.B * p.Hq * p.NB;
  const int blk = (int)blockIdx.x;
  if (blk < qblocks)
    bwd_prep_q_item<D>(p, tab, blk, st, st + BR * LS);
  else
    bwd_prep_k_item<D>(p, tab, blk - qblocks, st);
}

// ---------------------------------------------------------------------------------------------
// Per-wave dv (DV) or dk (!DV), the diagnostic alternative to bwd_dkdv_shared_item.
// Workgroup: (b, g, key-block pair), W waves; wave w takes the group's heads w, w+W, ...  The
// two gradients are separate kernels so that each holds one set of
// accumulators and has the registers to load the next query block's operands while it uses the
// current ones; the dv kernel needs neither dP nor dout in "c" layout.

template <int D, bool DV, bool SPLIT, bool SINGLE>
__global__ void __launch_bounds__(256, DV ? 2 : 1) bwd_dkdv_kernel(BwdParams p, RopeTable tab) {
  constexpr int NKK = D / 16;
  constexpr int NCB = D / 32;
  constexpr int T = BR * D;
  constexpr int RED = NCB * 16 * 64;  // floats of one accumulator set of a wave
  __shared__ float red[3][RED];
  // dv: the key block's operand, the same for every wave, is read from LDS at each step rather
  // than held in registers (two waves per SIMD leave no room for it beside two query blocks'
  // operands); dk keeps it in registers
  __shared__ bf16x8 kl[DV ? NKK * 64 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;
  // Work item: a pair of key blocks (kb, NB-1-kb), items renumbered so that one XCD runs one
  // K/V group; or (SINGLE) one key block, the heaviest first -- a causal key block kb is seen by
  // the NB - kb query blocks from kb on, so the grid runs kb = 0 first and the workgroups that
  // start last hold the lightest blocks -- renumbered the same way within each key block.
  const int n_hs = SPLIT ? p.HS : 1;          // head splits (SPLIT: more than one)
  const int per_kb = p.B * p.Hkv * n_hs;
  const int blk = SINGLE ? xcd_order(blockIdx.x % per_kb, per_kb) : xcd_order(blockIdx.x, gridDim.x);
  const int pair = SINGLE ? (int)(blockIdx.x / per_kb) : blk % p.n_pairs;
  const int hs = SPLIT ? (SINGLE ? blk : blk / p.n_pairs) % n_hs : 0;
  const int unit = (SINGLE ? blk : blk / p.n_pairs) / n_hs;  // b * Hkv + g
  const int g = unit % p.Hkv, b = unit / p.Hkv;
  const int c_off = hh * BR * 8 + l32 * 8;  // this lane's operand in a "c" tile (chunk 2kk + hh)

#pragma unroll 1
  for (int side = 0; side < (SINGLE ? 1 : 2); ++side) {
    const int kb = side == 0 ? pair : p.NB - 1 - pair;
    if (side == 1 && kb == pair) break;
    const size_t ktile = ((size_t)unit * p.NB + kb) * T;
    bf16x8 kf[NKK], vf[NKK];
    if constexpr (DV) {
      // operand kk of lane l at kl[64 kk + l]; the previous side's readers have passed the
      // barrier at the end of its reduction
      for (int i = threadIdx.x; i < NKK * 64; i += blockDim.x)
        kl[i] = ld16(p.kc + ktile + (i & 32) * BR / 4 + (i & 31) * 8 + (i >> 6) * 2 * BR * 8);
      __syncthreads();
    } else {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        kf[kk] = ld16(p.kc + ktile + c_off + kk * 2 * BR * 8);
        vf[kk] = ld16(p.vc + ktile + c_off + kk * 2 * BR * 8);
      }
    }
    const bool key_ok = kb * BR + l32 < p.S;
    const bool key_ok_all = (kb + 1) * BR <= p.S;  // every key of the block is a real one
    f32x16 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};

    // query-block operands, one set: as soon as an instruction has read its operand, the
    // register is reloaded with the next block's (see the dq kernel)
    bf16x8 qa[NKK], da[NKK], tb[2][NCB];
    f32x4 L[4], Dd[4];
    const int delta = p.q_pos0 - p.k_pos0;
    // the first query block with a row that sees a key of this block: 32 qb + 31 + delta >= 32 kb
    const int qb_lo = p.causal ? max(0, floor_div(BR * kb - delta, BR)) : 0;
    // per-lane byte offsets within a query block's tiles and row vectors
    const uint32_t v_c = 2u * c_off, v_t = 16u * (hh * D + l32), v_r = 16u * hh;
    for (int hc = wave + hs * p.W; hc < p.G; hc += p.W * n_hs) {
      const size_t qunit = (size_t)b * p.Hq + g * p.G + hc;
      // this head's run of query blocks as buffers (NB * T * 2 < 2^31 bytes)
      const uint32_t run_t = (uint32_t)p.NB * T * 2, run_r = (uint32_t)p.NB * BR * 4;
      const __amdgpu_buffer_rsrc_t qbuf = raw_buffer(p.qc + qunit * p.NB * T, run_t);
      const __amdgpu_buffer_rsrc_t dbuf = raw_buffer(p.dc + qunit * p.NB * T, run_t);
      const __amdgpu_buffer_rsrc_t tbuf = raw_buffer((DV ? p.dt : p.qt) + qunit * p.NB * T, run_t);
      const __amdgpu_buffer_rsrc_t lbuf = raw_buffer(p.l2 + qunit * p.NB * BR, run_r);
      const __amdgpu_buffer_rsrc_t ddbuf = raw_buffer(p.dd + qunit * p.NB * BR, run_r);
      auto ld_q = [&](int qb, int kk) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8, bld16(qbuf, v_c, (uint32_t)qb * T * 2 + kk * 2 * BR * 16));
      };
      auto ld_d = [&](int qb, int kk) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8, bld16(dbuf, v_c, (uint32_t)qb * T * 2 + kk * 2 * BR * 16));
      };
      auto ld_t = [&](int qb, int tt, int cb) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8, bld16(tbuf, v_t, (uint32_t)qb * T * 2 + (tt * 2 * D + 32 * cb) * 16));
      };
      // per-row lse and rowsum for this lane's rows 8c + 4hh + 0..3
      auto ld_rows = [&](int qb) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          L[c] = __builtin_bit_cast(f32x4, bld16(lbuf, v_r, (uint32_t)qb * BR * 4 + 32 * c));
          if (!DV) Dd[c] = __builtin_bit_cast(f32x4, bld16(ddbuf, v_r, (uint32_t)qb * BR * 4 + 32 * c));
        }
      };
      // P (dv) or dS (dk) of one step.  Key kb*32 + l32 is later than row qb*32 + r iff
      // l32 - r > rel, i.e. (r = res_row(v, hh)) iff 8(v/4) + v%4 < thr: one threshold per lane
      // and step, compared with constants and applied by selects, and only in the steps that
      // need it (a wave-uniform branch; a key past S masks every row, thr 32).
      auto probs = [&](const f32x16 &s, const f32x16 &dp, bool masked, int thr, bf16x8 (&op)[2])
          __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          u32x4 wv;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float x[2];
#pragma unroll
            for (int z = 0; z < 2; ++z) {
              const int v = 8 * tt + e + z;
              float pr = __builtin_amdgcn_exp2f(s[v] - L[v >> 2][v & 3]);
              if (masked) pr = 8 * (v >> 2) + (v & 3) < thr ? 0.f : pr;
              x[z] = DV ? pr : pr * (dp[v] - Dd[v >> 2][v & 3]);
            }
            wv[e / 2] = pack_bf16x2(x[0], x[1]);
          }
          op[tt] = __builtin_bit_cast(bf16x8, wv);
        }
      };
      auto step = [&](int qb, int qn) __attribute__((always_inline)) {
        f32x16 s = f32x16{}, dp = f32x16{};
        // (the LDS index goes through an empty asm so that the reads stay in the step)
        int ki = lane;
        if (DV) asm volatile("" : "+v"(ki));
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          s = bwd_mfma(qa[kk], DV ? kl[64 * kk + ki] : kf[kk], s);
          qa[kk] = ld_q(qn, kk);
          if (!DV) {
            dp = bwd_mfma(da[kk], vf[kk], dp);
            da[kk] = ld_d(qn, kk);
          }
        }
        const int rel = BR * (qb - kb) + delta;
        const bool masked = !key_ok_all || (p.causal && rel < BR - 1);  // wave-uniform
        const int thr = !key_ok ? 32 : (p.causal && rel < BR - 1) ? l32 - 4 * hh - rel : 0;
        bf16x8 op[2];
        if (masked)
          probs(s, dp, true, thr, op);
        else
          probs(s, dp, false, thr, op);
        ld_rows(qn);
        // dv += P^T dO, dk += dS^T (q'/sqrt(D))
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            acc[cb] = bwd_mfma(op[tt], tb[tt][cb], acc[cb]);
            tb[tt][cb] = ld_t(qn, tt, cb);
          }
      };
      // from the last query block down, so that the workgroups of a group sweep the same
      // query tiles at about the same time; the clamped index re-reads the last block
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        qa[kk] = ld_q(p.NB - 1, kk);
        if (!DV) da[kk] = ld_d(p.NB - 1, kk);
      }
      ld_rows(p.NB - 1);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) tb[tt][cb] = ld_t(p.NB - 1, tt, cb);
      // the first operands are in before the loop, so that the waits inside it count only the
      // loop's own loads (vmcnt(0), the other counters untouched)
      __builtin_amdgcn_s_waitcnt(0x0F70);
      for (int qb = p.NB - 1; qb >= qb_lo; --qb) step(qb, max(qb - 1, qb_lo));
    }

    // add the waves' sums into wave 0
    if (wave > 0) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[wave - 1][(cb * 16 + v) * 64 + lane] = acc[cb][v];
    }
    __syncthreads();
    if (wave == 0) {
      for (int w = 1; w < p.W; ++w)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[cb][v] += red[w - 1][(cb * 16 + v) * 64 + lane];
      // result lane = column 32 cb + l32, register v = key 8(v/4) + 4 hh + v%4 of the block
      if constexpr (SPLIT) {
        // this head split's partial sums (dk' not yet rotated back), for the reduction kernel
        float *part = p.part + (((size_t)(DV ? n_hs : 0) + hs) * p.B * p.Hkv + unit) * p.NB * BR * D;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kb * BR + res_row(v, hh);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) part[(size_t)key * D + 32 * cb + l32] = acc[cb][v];
        }
      } else {
      // dk' -> dk: rotate the pair (column i, i + D/2) back by the key's angle
      if (!DV) {
#pragma unroll
        for (int cb = 0; cb < NCB / 2; ++cb) {
          const double rev = tab.rev[32 * cb + l32];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kb * BR + res_row(v, hh);
            const float t = turn_fraction(p.k_pos0 + key, rev);
            const float sn = __builtin_amdgcn_sinf(t), cs = __builtin_amdgcn_cosf(t);
            const float x = acc[cb][v], y = acc[cb + NCB / 2][v];
            acc[cb][v] = x * cs + y * sn;
            acc[cb + NCB / 2][v] = y * cs - x * sn;
          }
        }
      }
      __bf16 *dst0 = DV ? p.dv : p.dk;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kb * BR + res_row(v, hh);
        if (key < p.S) {
          const size_t dst = (((size_t)b * p.S + key) * p.Hkv + g) * D;
          // dk of the adjacent-pair form goes back to the original dim order; dv is never reordered
          const int il = DV ? 0 : tab.interleaved;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) dst0[dst + rope_src_dim(32 * cb + l32, D / 2, il)] = (__bf16)acc[cb][v];
        }
      }
      }
    }
    __syncthreads();  // the reduction slots are reused by the second block
  }
}

// ---------------------------------------------------------------------------------------------
// Per-wave dq, the diagnostic alternative to bwd_dq_shared_item (ATTN_BWD_DQ=regs).  One wave
// per (b, h, query-block pair), or per query block with SINGLE.

template <int D, bool SINGLE>
__global__ void __launch_bounds__(64, D == 64 ? 2 : 1) bwd_dq_kernel(BwdParams p, RopeTable tab) {
  constexpr int NKK = D / 16;
  constexpr int NCB = D / 32;
  constexpr int T = BR * D;
  const int lane = threadIdx.x;
  const int l32 = lane & 31, hh = lane >> 5;
  // Work item: a pair of query blocks (qb, NB-1-qb), items renumbered so that one XCD runs one
  // K/V group; or (SINGLE) one query block, the heaviest first (causal query block qb sees
  // qb + 1 key blocks, so the grid runs qb = NB-1 first), renumbered the same way within each.
  const int per_qb = p.B * p.Hq;
  const int blk = SINGLE ? xcd_order(blockIdx.x % per_qb, per_qb) : xcd_order(blockIdx.x, gridDim.x);
  const int pair = SINGLE ? p.NB - 1 - (int)(blockIdx.x / per_qb) : blk % p.n_pairs;
  const int qunit = SINGLE ? blk : blk / p.n_pairs;  // b * Hq + h
  const int h = qunit % p.Hq, b = qunit / p.Hq;
  const int g = h / p.G;
  const size_t kunit = (size_t)b * p.Hkv + g;
  const int c_off = hh * BR * 8 + l32 * 8;

  for (int side = 0; side < (SINGLE ? 1 : 2); ++side) {
    const int qb = side == 0 ? pair : p.NB - 1 - pair;
    if (side == 1 && qb == pair) break;
    const size_t qtile = ((size_t)qunit * p.NB + qb) * T;
    bf16x8 qf[NKK], df[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qf[kk] = ld16(p.qc + qtile + c_off + kk * 2 * BR * 8);
      df[kk] = ld16(p.dc + qtile + c_off + kk * 2 * BR * 8);
    }
    // this lane's query: row l32 of the block
    const float Lq = p.l2[((size_t)qunit * p.NB + qb) * BR + l32];
    const float Dq = p.dd[((size_t)qunit * p.NB + qb) * BR + l32];
    f32x16 dq[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) dq[cb] = f32x16{};
    const int delta = p.q_pos0 - p.k_pos0;
    // key blocks with a key some row of this block sees: 32 kb <= 32 qb + 31 + delta
    const int kb_end = p.causal ? min(p.NB, max(0, floor_div(BR * qb + BR - 1 + delta, BR) + 1)) : p.NB;
    // key-block operands, one set: as soon as an MFMA has read its operand, the register is
    // reloaded with the next block's (the index is clamped, so the last step re-reads its own
    // block instead of branching)
    bf16x8 ka[NKK], va[NKK], kt[2][NCB];
    // this K/V head's run of key blocks as buffers (NB * T * 2 < 2^31 bytes), per-lane byte offsets
    const uint32_t run_t = (uint32_t)p.NB * T * 2;
    const __amdgpu_buffer_rsrc_t kbuf = raw_buffer(p.kc + kunit * p.NB * T, run_t);
    const __amdgpu_buffer_rsrc_t vbuf = raw_buffer(p.vc + kunit * p.NB * T, run_t);
    const __amdgpu_buffer_rsrc_t tbuf = raw_buffer(p.kt + kunit * p.NB * T, run_t);
    const uint32_t v_c = 2u * c_off, v_t = 16u * (hh * D + l32);
    auto ld_k = [&](int kb, int kk) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8, bld16(kbuf, v_c, (uint32_t)kb * T * 2 + kk * 2 * BR * 16));
    };
    auto ld_v = [&](int kb, int kk) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8, bld16(vbuf, v_c, (uint32_t)kb * T * 2 + kk * 2 * BR * 16));
    };
    auto ld_t = [&](int kb, int tt, int cb) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x8, bld16(tbuf, v_t, (uint32_t)kb * T * 2 + (tt * 2 * D + 32 * cb) * 16));
    };
    // P and dS of one step; the element mask only in the steps that need it (a wave-uniform
    // branch), as one threshold per lane compared with constants and applied by selects
    auto probs = [&](const f32x16 &st, const f32x16 &dpt, bool masked, int thr, int kend, bf16x8 (&sa)[2])
        __attribute__((always_inline)) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        u32x4 ws;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float sv[2];
#pragma unroll
          for (int z = 0; z < 2; ++z) {
            const int v = 8 * tt + e + z;
            float pr = __builtin_amdgcn_exp2f(st[v] - Lq);
            if (masked) pr = ((8 * (v >> 2) + (v & 3) > thr) | (8 * (v >> 2) + (v & 3) >= kend)) ? 0.f : pr;
            sv[z] = pr * (dpt[v] - Dq);
          }
          ws[e / 2] = pack_bf16x2(sv[0], sv[1]);
        }
        sa[tt] = __builtin_bit_cast(bf16x8, ws);
      }
    };
    auto step = [&](int kb, int kn) __attribute__((always_inline)) {
      f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        st = bwd_mfma(ka[kk], qf[kk], st);
        ka[kk] = ld_k(kn, kk);
        dpt = bwd_mfma(va[kk], df[kk], dpt);
        va[kk] = ld_v(kn, kk);
      }
      // key kb*32 + k is later than row qb*32 + l32 iff k - l32 > rel, i.e. (k = res_row(v, hh))
      // iff 8(v/4) + v%4 > thr.  Keys past S: those of the last block from S - 32 kb on.
      const int rel = BR * (qb - kb) + delta;
      const bool masked = (p.causal && rel < BR - 1) || (kb + 1) * BR > p.S;  // wave-uniform
      const int thr = (p.causal && rel < BR - 1) ? rel + l32 - 4 * hh : 27;
      const int kend = p.S - kb * BR - 4 * hh;  // key 8(v/4) + v%4 + 4hh < S iff 8(v/4) + v%4 < kend
      bf16x8 sa[2];
      if (masked)
        probs(st, dpt, true, thr, kend, sa);
      else
        probs(st, dpt, false, thr, kend, sa);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          dq[cb] = bwd_mfma(sa[tt], kt[tt][cb], dq[cb]);
          kt[tt][cb] = ld_t(kn, tt, cb);
        }
    };
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      ka[kk] = ld_k(0, kk);
      va[kk] = ld_v(0, kk);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) kt[tt][cb] = ld_t(0, tt, cb);
    // the first operands are in before the loop, so that the waits inside it count only the
    // loop's own loads (vmcnt(0), the other counters untouched).  Each step also ends with every
    // load in: letting them run on (24 KiB of loads in flight per wave) keeps the same time at
    // 2K keys but costs 20% at 32K, where the key tiles of a K/V head no longer fit an XCD's L2
    // and the waves of a head, drifting apart, stop sharing them there.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    for (int kb = 0; kb < kb_end; ++kb) {
      step(kb, min(kb + 1, kb_end - 1));
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    // result lane = column 32 cb + l32, register v = query 8(v/4) + 4 hh + v%4 of the block
#pragma unroll
    for (int cb = 0; cb < NCB / 2; ++cb) {
      const double rev = tab.rev[32 * cb + l32];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = qb * BR + res_row(v, hh);
        const float t = turn_fraction(p.q_pos0 + row, rev);
        const float sn = __builtin_amdgcn_sinf(t), cs = __builtin_amdgcn_cosf(t);
        const float x = dq[cb][v] * p.inv_sqrt_d, y = dq[cb + NCB / 2][v] * p.inv_sqrt_d;
        dq[cb][v] = x * cs + y * sn;
        dq[cb + NCB / 2][v] = y * cs - x * sn;
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = qb * BR + res_row(v, hh);
      if (row < p.S) {
        const size_t dst = (((size_t)b * p.S + row) * p.Hq + h) * D;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) p.dq[dst + rope_src_dim(32 * cb + l32, D / 2, tab.interleaved)] = (__bf16)dq[cb][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dq with the key blocks shared by the waves of a workgroup: W = min(G, 4) query heads of a K/V
// group (pass * W + w % W) times 4 / W consecutive query blocks of them (W = 3: three waves on
// one block).  Work items: groups of query blocks, the heaviest first, renumbered within each
// rank so that one XCD runs one K/V group.  Each key block's three tiles (rotated keys in "c"
// and "t" layouts, values in "c" layout, 3 * 32 * D bf16) are copied once per workgroup from
// L2 into LDS (16-byte loads straight into LDS, the waves taking turns) and every wave reads
// its MFMA operands there, so the path from L2 into the CU carries each tile once per
// workgroup instead of once per wave; a wave skips the key blocks its query block does not
// see.  Double-buffered: the copy of block kb+1 runs during block kb; one barrier per block.
// Same arithmetic, operand layouts, visibility and masks as bwd_dq_kernel.

__device__ __forceinline__ void bwd_lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, char *lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)lds_base, 16, voff, soff, 0, 0);
}

// LDS of one key-block buffer of the shared dq kernel: [kc | vc | kt]
template <int D>
constexpr int bwd_dq_buf_bytes() {
  return 3 * BR * D * 2;
}

// Query blocks per workgroup of the shared dq kernel with W heads: four waves in all where W
// divides four (one head: four consecutive query blocks), else one block.
template <int W>
constexpr int bwd_dq_qw() {
  return W == 1 ? 4 : W == 2 ? 2 : 1;
}

// work item blk: W heads times QW consecutive query blocks, the top one NB - 1 - QW (blk /
// per_qg) (the heaviest first); wave w serves head w % W of its pass and query block
// top - w / W; the two key-block buffers kbuf0, kbuf1
template <int D, int W>
__device__ __forceinline__ void bwd_dq_shared_item(const BwdParams &p, const RopeTable &tab, int blk, char *kbuf0,
                                                   char *kbuf1) {
  constexpr int NKK = D / 16;
  constexpr int NCB = D / 32;
  constexpr int T = BR * D;
  constexpr int TB = T * 2;               // bytes of one tile
  constexpr int NPART = TB / 1024;        // 1 KiB copy instructions per tile
  constexpr int QW = bwd_dq_qw<W>();
  constexpr int NW = W * QW;              // waves
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;
  const int passes = (p.G + W - 1) / W;
  const int per_qg = p.B * p.Hkv * passes;
  const int qb_top = p.NB - 1 - QW * (blk / per_qg);
  const int qb_raw = qb_top - wave / W;
  const bool has_qb = qb_raw >= 0;
  const int qb = has_qb ? qb_raw : 0;  // (a wave past the first block computes on block 0 and writes nothing)
  const int item = xcd_order(blk % per_qg, per_qg);
  const int pass = item % passes;
  const int kunit = item / passes;  // b * Hkv + g
  const int g = kunit % p.Hkv, b = kunit / p.Hkv;
  const int hc = pass * W + wave % W;  // head of the group this wave serves (none past G)
  const bool has_head = hc < p.G && has_qb;
  const int h = g * p.G + (hc < p.G ? hc : 0);
  const size_t qunit = (size_t)b * p.Hq + h;
  const int c_off = hh * BR * 8 + l32 * 8;
  const int delta = p.q_pos0 - p.k_pos0;

  const size_t qtile = (qunit * p.NB + qb) * T;
  bf16x8 qf[NKK], df[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qf[kk] = ld16(p.qc + qtile + c_off + kk * 2 * BR * 8);
    df[kk] = ld16(p.dc + qtile + c_off + kk * 2 * BR * 8);
  }
  // this lane's query: row l32 of the block
  const float Lq = p.l2[(qunit * p.NB + qb) * BR + l32];
  const float Dq = p.dd[(qunit * p.NB + qb) * BR + l32];
  f32x16 dq[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) dq[cb] = f32x16{};
  // key blocks with a key some row of block q sees: 32 kb <= 32 q + 31 + delta
  auto kb_end_of = [&](int q) __attribute__((always_inline)) {
    return p.causal ? min(p.NB, max(0, floor_div(BR * q + BR - 1 + delta, BR) + 1)) : p.NB;
  };
  const int kb_end = has_qb ? kb_end_of(qb) : 0;  // this wave's
  const int wg_kb_end = kb_end_of(qb_top);        // the workgroup's (its top block sees the most)

  // this K/V head's run of key blocks as buffers (NB * T * 2 < 2^31 bytes)
  const uint32_t run_t = (uint32_t)p.NB * TB;
  const __amdgpu_buffer_rsrc_t kcb = raw_buffer(p.kc + (size_t)kunit * p.NB * T, run_t);
  const __amdgpu_buffer_rsrc_t vcb = raw_buffer(p.vc + (size_t)kunit * p.NB * T, run_t);
  const __amdgpu_buffer_rsrc_t ktb = raw_buffer(p.kt + (size_t)kunit * p.NB * T, run_t);
  // this wave's share of the copies of key block kb into dst: KiB wave, wave + W, ... of each
  // tile (the tile, and so the buffer resource, known at compile time)
  auto copy_block = [&](int kb, char *dst) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const __amdgpu_buffer_rsrc_t r = t == 0 ? kcb : t == 1 ? vcb : ktb;
#pragma unroll
      for (int i = 0; i < (NPART + NW - 1) / NW; ++i) {
        const int part = wave + NW * i;
        if (NPART % NW == 0 || part < NPART)
          bwd_lds_dma16(r, 16u * lane, (uint32_t)kb * TB + part * 1024, dst + t * TB + part * 1024);
      }
    }
  };
  const int v_c = 2 * c_off, v_t = 16 * (hh * D + l32);
  auto step = [&](int kb, const char *src) __attribute__((always_inline)) {
    if (kb >= kb_end) return;  // no key of block kb is seen by this wave's block
    f32x16 st = f32x16{}, dpt = f32x16{};
    // the score products' operands are read from LDS first, all of them, then used
    bf16x8 ka[NKK], va[NKK], kt[2][NCB];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      ka[kk] = *reinterpret_cast<const bf16x8 *>(src + v_c + kk * 2 * BR * 16);
      va[kk] = *reinterpret_cast<const bf16x8 *>(src + TB + v_c + kk * 2 * BR * 16);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      st = bwd_mfma(ka[kk], qf[kk], st);
      dpt = bwd_mfma(va[kk], df[kk], dpt);
    }
    // the gradient product's operands are read while the softmax arithmetic runs
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        kt[tt][cb] = *reinterpret_cast<const bf16x8 *>(src + 2 * TB + v_t + (tt * 2 * D + 32 * cb) * 16);
    // key kb*32 + k is later than row qb*32 + l32 iff k - l32 > rel, i.e. (k = res_row(v, hh))
    // iff 8(v/4) + v%4 > thr.  Keys past S: those of the last block from S - 32 kb on.
    const int rel = BR * (qb - kb) + delta;
    const bool masked = (p.causal && rel < BR - 1) || (kb + 1) * BR > p.S;  // wave-uniform
    const int thr = (p.causal && rel < BR - 1) ? rel + l32 - 4 * hh : 27;
    const int kend = p.S - kb * BR - 4 * hh;
    bf16x8 sa[2];
    auto probs = [&](bool msk) __attribute__((always_inline)) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        u32x4 ws;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float sv[2];
#pragma unroll
          for (int z = 0; z < 2; ++z) {
            const int v = 8 * tt + e + z;
            float pr = __builtin_amdgcn_exp2f(st[v] - Lq);
            if (msk) pr = ((8 * (v >> 2) + (v & 3) > thr) | (8 * (v >> 2) + (v & 3) >= kend)) ? 0.f : pr;
            sv[z] = pr * (dpt[v] - Dq);
          }
          ws[e / 2] = pack_bf16x2(sv[0], sv[1]);
        }
        sa[tt] = __builtin_bit_cast(bf16x8, ws);
      }
    };
    if (masked)
      probs(true);
    else
      probs(false);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        dq[cb] = bwd_mfma(sa[tt], kt[tt][cb], dq[cb]);
  };
  // Block kb sits in buffer kb % 2.  Before block kb: its copy is in (issued a block earlier)
  // and every wave has finished block kb - 1; then the copy of block kb + 1 goes into the
  // buffer block kb - 1 used.
  if (wg_kb_end > 0) copy_block(0, kbuf0);
  for (int kb = 0; kb < wg_kb_end; kb += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (kb + 1 < wg_kb_end) copy_block(kb + 1, kbuf1);
    step(kb, kbuf0);
    if (kb + 1 < wg_kb_end) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (kb + 2 < wg_kb_end) copy_block(kb + 2, kbuf0);
      step(kb + 1, kbuf1);
    }
  }
  if (!has_head) return;
  // result lane = column 32 cb + l32, register v = query 8(v/4) + 4 hh + v%4 of the block
#pragma unroll
  for (int cb = 0; cb < NCB / 2; ++cb) {
    const double rev = tab.rev[32 * cb + l32];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = qb * BR + res_row(v, hh);
      const float t = turn_fraction(p.q_pos0 + row, rev);
      const float sn = __builtin_amdgcn_sinf(t), cs = __builtin_amdgcn_cosf(t);
      const float x = dq[cb][v] * p.inv_sqrt_d, y = dq[cb + NCB / 2][v] * p.inv_sqrt_d;
      dq[cb][v] = x * cs + y * sn;
      dq[cb + NCB / 2][v] = y * cs - x * sn;
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = qb * BR + res_row(v, hh);
    if (row < p.S) {
      const size_t dst = (((size_t)b * p.S + row) * p.Hq + h) * D;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) p.dq[dst + rope_src_dim(32 * cb + l32, D / 2, tab.interleaved)] = (__bf16)dq[cb][v];
    }
  }
}

template <int D, int W>
__global__ void __launch_bounds__(64 * W * bwd_dq_qw<W>()) bwd_dq_shared_kernel(BwdParams p, RopeTable tab) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * bwd_dq_buf_bytes<D>()];
  bwd_dq_shared_item<D, W>(p, tab, (int)blockIdx.x, lds, lds + bwd_dq_buf_bytes<D>());
}

// ---------------------------------------------------------------------------------------------
// dv (DV) or dk (!DV) with the query blocks shared by consecutive key blocks.  Workgroup: KW = 4
// waves, wave w key block kg * KW + w of K/V head (b, g); the group's query heads of this head
// split (hs, hs + HS, ...) one after another, and for each the query blocks from the last one
// down.  Each query block's tiles (scaled rotated queries in "c" layout, dout in "c" layout for
// dk, queries ("t") for dk or dout ("t") for dv) are copied once per workgroup from L2 into LDS
// (16-byte loads straight into LDS, the waves taking turns, double-buffered, one barrier per
// block), with the block's 32 lse and rowsum values, and every wave reads its MFMA operands and
// those values there (read from global memory at the step that needs them, their latency showed
// in every step).  A wave skips the blocks that see none of its keys.  Its sums over the heads
// stay in its registers: dk is rotated back and written (or, with head splits, left as fp32
// partials for bwd_part_reduce).  Work items: key-block groups, the heaviest (kg = 0) first,
// renumbered within each so that one XCD runs one K/V head.

constexpr int KW = 4;  // key blocks (waves) per workgroup

// Gradients one work item computes: dk, dv, or both from one pass (the probabilities and dS of
// a step computed once for the two products; head_dim 64, where both accumulator sets fit).
enum BwdKvKind { kKvDk = 0, kKvDv = 1, kKvBoth = 2 };

// tiles per query block, in LDS order: [qc | dc | qt] (dk), [qc | dt] (dv), [qc | dc | qt | dt]
template <int KIND>
constexpr int bwd_kv_tiles() {
  return KIND == kKvDk ? 3 : KIND == kKvDv ? 2 : 4;
}

// LDS of one query-block buffer: the tiles, then 1 KiB for the block's lse rows and 1 KiB for
// its rowsums
template <int D, int KIND>
constexpr int bwd_kv_buf_bytes() {
  return bwd_kv_tiles<KIND>() * BR * D * 2 + 2048;
}

// work item blk (key group blk / per_kg, the heaviest first) with the two buffers qbuf0, qbuf1
template <int D, int KIND, bool SPLIT>
__device__ __forceinline__ void bwd_dkdv_shared_item(const BwdParams &p, const RopeTable &tab, int blk, char *qbuf0,
                                                     char *qbuf1) {
  constexpr bool DO_K = KIND != kKvDv, DO_V = KIND != kKvDk;
  constexpr int NKK = D / 16;
  constexpr int NCB = D / 32;
  constexpr int T = BR * D;
  constexpr int TB = T * 2;             // bytes of one tile
  constexpr int NPART = TB / 1024;      // 1 KiB copy instructions per tile
  constexpr int NT = bwd_kv_tiles<KIND>();
  constexpr int RB = NT * TB;           // then the lse and rowsum rows
  constexpr int T_Q = 2, T_D = KIND == kKvDv ? 1 : 3;  // tiles of the "t" operands: qt, dt
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l32 = lane & 31, hh = lane >> 5;
  const int n_hs = SPLIT ? p.HS : 1;
  const int per_kg = p.B * p.Hkv * n_hs;
  const int kg = blk / per_kg;
  const int item = xcd_order(blk % per_kg, per_kg);
  const int hs = SPLIT ? item % n_hs : 0;
  const int unit = item / n_hs;  // b * Hkv + g
  const int g = unit % p.Hkv, b = unit / p.Hkv;
  const int kb = kg * KW + wave;
  const bool has_kb = kb < p.NB;
  const int kbc = has_kb ? kb : p.NB - 1;  // (a wave past the last block computes on the last one and writes nothing)
  const int c_off = hh * BR * 8 + l32 * 8;
  const int delta = p.q_pos0 - p.k_pos0;
  const size_t ktile = ((size_t)unit * p.NB + kbc) * T;
  bf16x8 kf[NKK], vf[DO_K ? NKK : 1];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    kf[kk] = ld16(p.kc + ktile + c_off + kk * 2 * BR * 8);
    if constexpr (DO_K) vf[kk] = ld16(p.vc + ktile + c_off + kk * 2 * BR * 8);
  }
  const bool key_ok = kbc * BR + l32 < p.S;
  const bool key_ok_all = (kbc + 1) * BR <= p.S;
  // the first query block with a row that sees a key of block kb: 32 qb + 31 + delta >= 32 kb
  auto qb_lo_of = [&](int k) __attribute__((always_inline)) {
    return p.causal ? max(0, floor_div(BR * k - delta, BR)) : 0;
  };
  const int my_qb_lo = qb_lo_of(kbc);
  const int wg_qb_lo = qb_lo_of(kg * KW);  // the workgroup's first key block sees the most
  f32x16 acc_k[DO_K ? NCB : 1], acc_v[DO_V ? NCB : 1];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    if constexpr (DO_K) acc_k[cb] = f32x16{};
    if constexpr (DO_V) acc_v[cb] = f32x16{};
  }
  const int v_c = 2 * c_off, v_t = 16 * (hh * D + l32), v_r = 16 * hh;
  const uint32_t run_t = (uint32_t)p.NB * TB, run_r = (uint32_t)p.NB * BR * 4;

  for (int hc = hs; hc < p.G; hc += n_hs) {
    const size_t qunit = (size_t)b * p.Hq + g * p.G + hc;
    const __amdgpu_buffer_rsrc_t qcb = raw_buffer(p.qc + qunit * p.NB * T, run_t);
    const __amdgpu_buffer_rsrc_t dcb = raw_buffer(p.dc + qunit * p.NB * T, run_t);
    const __amdgpu_buffer_rsrc_t qtb = raw_buffer(p.qt + qunit * p.NB * T, run_t);
    const __amdgpu_buffer_rsrc_t dtb = raw_buffer(p.dt + qunit * p.NB * T, run_t);
    const __amdgpu_buffer_rsrc_t lbuf = raw_buffer(p.l2 + qunit * p.NB * BR, run_r);
    const __amdgpu_buffer_rsrc_t ddbuf = raw_buffer(p.dd + qunit * p.NB * BR, run_r);
    // this wave's share of the copies of query block qb into dst: KiB wave, wave + KW, ... of
    // each tile (the tile, and so the buffer resource, known at compile time)
    auto copy_block = [&](int qb, char *dst) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const __amdgpu_buffer_rsrc_t r = t == 0 ? qcb : t == T_D ? dtb : t == T_Q ? qtb : dcb;
#pragma unroll
        for (int i = 0; i < (NPART + KW - 1) / KW; ++i) {
          const int part = wave + KW * i;
          if (NPART % KW == 0 || part < NPART)
            bwd_lds_dma16(r, 16u * lane, (uint32_t)qb * TB + part * 1024, dst + t * TB + part * 1024);
        }
      }
      // the block's 32 lse (and rowsum) values: 128 bytes from lanes 0..7; the other lanes'
      // offsets lie past the buffer's end, so they read nothing
      const uint32_t roff = lane < 8 ? (uint32_t)qb * BR * 4 + 16u * lane : 0x80000000u;
      if (wave == KW - 1) bwd_lds_dma16(lbuf, roff, 0, dst + RB);
      if (DO_K && wave == KW - 2) bwd_lds_dma16(ddbuf, roff, 0, dst + RB + 1024);
    };
    auto step = [&](int qb, const char *src) __attribute__((always_inline)) {
      if (qb < my_qb_lo) return;  // no key of this wave's block is seen by this query block
      bf16x8 qa[NKK], da[DO_K ? NKK : 1];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        qa[kk] = *reinterpret_cast<const bf16x8 *>(src + v_c + kk * 2 * BR * 16);
        if constexpr (DO_K) da[kk] = *reinterpret_cast<const bf16x8 *>(src + TB + v_c + kk * 2 * BR * 16);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s = bwd_mfma(qa[kk], kf[kk], s);
        if constexpr (DO_K) dp = bwd_mfma(da[kk], vf[kk], dp);
      }
      // lse and rowsum of this lane's rows 8c + 4hh + 0..3
      f32x4 L[4], Dd[DO_K ? 4 : 1];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        L[c] = *reinterpret_cast<const f32x4 *>(src + RB + v_r + 32 * c);
        if constexpr (DO_K) Dd[c] = *reinterpret_cast<const f32x4 *>(src + RB + 1024 + v_r + 32 * c);
      }
      // the "t" operands of the gradient products: queries (dk), dout (dv)
      bf16x8 tq[DO_K ? 2 : 1][NCB], td[DO_V ? 2 : 1][NCB];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          if constexpr (DO_K) tq[tt][cb] = *reinterpret_cast<const bf16x8 *>(src + T_Q * TB + v_t + (tt * 2 * D + 32 * cb) * 16);
          if constexpr (DO_V) td[tt][cb] = *reinterpret_cast<const bf16x8 *>(src + T_D * TB + v_t + (tt * 2 * D + 32 * cb) * 16);
        }
      // key kb*32 + l32 is later than row qb*32 + r iff l32 - r > rel, i.e. (r = res_row(v, hh))
      // iff 8(v/4) + v%4 < thr: one threshold per lane, applied by selects in the steps that
      // need it (a key past S masks every row, thr 32)
      const int rel = BR * (qb - kbc) + delta;
      const bool masked = !key_ok_all || (p.causal && rel < BR - 1);  // wave-uniform
      const int thr = !key_ok ? 32 : (p.causal && rel < BR - 1) ? l32 - 4 * hh - rel : 0;
      bf16x8 op_p[DO_V ? 2 : 1], op_s[DO_K ? 2 : 1];  // P and dS, packed as A operands
      auto probs = [&](bool msk) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          u32x4 wp, ws;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float xp[2], xs[2];
#pragma unroll
            for (int z = 0; z < 2; ++z) {
              const int v = 8 * tt + e + z;
              float pr = __builtin_amdgcn_exp2f(s[v] - L[v >> 2][v & 3]);
              if (msk) pr = 8 * (v >> 2) + (v & 3) < thr ? 0.f : pr;
              xp[z] = pr;
              if constexpr (DO_K) xs[z] = pr * (dp[v] - Dd[v >> 2][v & 3]);
            }
            if constexpr (DO_V) wp[e / 2] = pack_bf16x2(xp[0], xp[1]);
            if constexpr (DO_K) ws[e / 2] = pack_bf16x2(xs[0], xs[1]);
          }
          if constexpr (DO_V) op_p[tt] = __builtin_bit_cast(bf16x8, wp);
          if constexpr (DO_K) op_s[tt] = __builtin_bit_cast(bf16x8, ws);
        }
      };
      if (masked)
        probs(true);
      else
        probs(false);
      // dv += P^T dO, dk += dS^T (q'/sqrt(D))
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          if constexpr (DO_V) acc_v[cb] = bwd_mfma(op_p[tt], td[tt][cb], acc_v[cb]);
          if constexpr (DO_K) acc_k[cb] = bwd_mfma(op_s[tt], tq[tt][cb], acc_k[cb]);
        }
    };
    // query block qb sits in buffer qb % 2 ... counted from the top: block NB-1-j in buffer j % 2.
    // Before each block: its copy is in and every wave has finished the previous block; then
    // the copy of the next block goes into the buffer the previous one used.
    __syncthreads();  // the previous head's last block is no longer read
    if (p.NB - 1 >= wg_qb_lo) copy_block(p.NB - 1, qbuf0);
    for (int qb = p.NB - 1; qb >= wg_qb_lo; qb -= 2) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (qb - 1 >= wg_qb_lo) copy_block(qb - 1, qbuf1);
      step(qb, qbuf0);
      if (qb - 1 >= wg_qb_lo) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (qb - 2 >= wg_qb_lo) copy_block(qb - 2, qbuf0);
        step(qb - 1, qbuf1);
      }
    }
  }
  if (!has_kb) return;
  // result lane = column 32 cb + l32, register v = key 8(v/4) + 4 hh + v%4 of the block; dk is
  // rotated back, dv written as is (or, with head splits, both left as fp32 partials)
  auto finish = [&](auto is_v, f32x16 (&acc)[NCB]) __attribute__((always_inline)) {
    constexpr bool DV = decltype(is_v)::value;
    if constexpr (SPLIT) {
      float *part = p.part + (((size_t)(DV ? n_hs : 0) + hs) * p.B * p.Hkv + unit) * p.NB * BR * D;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kb * BR + res_row(v, hh);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) part[(size_t)key * D + 32 * cb + l32] = acc[cb][v];
      }
    } else {
      if (!DV) {
#pragma unroll
        for (int cb = 0; cb < NCB / 2; ++cb) {
          const double rev = tab.rev[32 * cb + l32];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kb * BR + res_row(v, hh);
            const float t = turn_fraction(p.k_pos0 + key, rev);
            const float sn = __builtin_amdgcn_sinf(t), cs = __builtin_amdgcn_cosf(t);
            const float x = acc[cb][v], y = acc[cb + NCB / 2][v];
            acc[cb][v] = x * cs + y * sn;
            acc[cb + NCB / 2][v] = y * cs - x * sn;
          }
        }
      }
      __bf16 *dst0 = DV ? p.dv : p.dk;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kb * BR + res_row(v, hh);
        if (key < p.S) {
          const size_t dst = (((size_t)b * p.S + key) * p.Hkv + g) * D;
          const int il = DV ? 0 : tab.interleaved;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) dst0[dst + rope_src_dim(32 * cb + l32, D / 2, il)] = (__bf16)acc[cb][v];
        }
      }
    }
  };
  if constexpr (DO_V) finish(std::true_type{}, acc_v);
  if constexpr (DO_K) finish(std::false_type{}, acc_k);
}

// KINDS, a set of work-item kinds in one launch: 1 dk, 2 dv, 4 dq (the shared dq kernel with KW
// heads per workgroup), 8 dk and dv together (head_dim 64).  With more than one kind the work
// items go by level, heaviest first: level j holds the dk and dv items of key group j and the
// dq items of query blocks NB-1-4j down to NB-4-4j, which see as many key blocks as key group
// j sees query blocks; within a level the items with more products per step come first.  The
// light items of every kind then fill the CUs as the heavy ones end.
template <int D, int KINDS>
constexpr int bwd_kv_lds_bytes() {
  int b = 0;
  if (KINDS & 1) b = bwd_kv_buf_bytes<D, kKvDk>();
  if ((KINDS & 8) && bwd_kv_buf_bytes<D, kKvBoth>() > b) b = bwd_kv_buf_bytes<D, kKvBoth>();
  if ((KINDS & 2) && bwd_kv_buf_bytes<D, kKvDv>() > b) b = bwd_kv_buf_bytes<D, kKvDv>();
  if ((KINDS & 4) && bwd_dq_buf_bytes<D>() > b) b = bwd_dq_buf_bytes<D>();
  return b;
}

template <int D, bool SPLIT, int KINDS>
__global__ void __launch_bounds__(64 * KW) __attribute__((amdgpu_waves_per_eu(2)))  // <= 256 registers
bwd_dkdv_shared_kernel(BwdParams p, RopeTable tab) {
  constexpr int BUF = bwd_kv_lds_bytes<D, KINDS>();
  __shared__ __attribute__((aligned(1024))) char lds[2 * BUF];
  constexpr int NKV = ((KINDS & 1) ? 1 : 0) + ((KINDS & 2) ? 1 : 0) + ((KINDS & 8) ? 1 : 0);
  if constexpr (NKV == 1 && (KINDS & 4) == 0) {  // one kind: the block is the item
    constexpr int KIND = (KINDS & 1) ? kKvDk : (KINDS & 2) ? kKvDv : kKvBoth;
    bwd_dkdv_shared_item<D, KIND, SPLIT>(p, tab, (int)blockIdx.x, lds, lds + BUF);
    return;
  }
  const int per_kg = p.B * p.Hkv * (SPLIT ? p.HS : 1);
  const int per_q = (KINDS & 4) ? p.B * p.Hkv * ((p.G + KW - 1) / KW) : 0;  // dq items per query block
  const int L = NKV * per_kg + KW * per_q;                                 // items per level
  const int lvl = (int)blockIdx.x / L;
  int r = (int)blockIdx.x % L;
  if constexpr ((KINDS & 1) != 0) {
    if (r < per_kg) {
      bwd_dkdv_shared_item<D, kKvDk, SPLIT>(p, tab, lvl * per_kg + r, lds, lds + bwd_kv_buf_bytes<D, kKvDk>());
      return;
    }
    r -= per_kg;
  }
  if constexpr ((KINDS & 8) != 0) {
    if (r < per_kg) {
      bwd_dkdv_shared_item<D, kKvBoth, SPLIT>(p, tab, lvl * per_kg + r, lds, lds + bwd_kv_buf_bytes<D, kKvBoth>());
      return;
    }
    r -= per_kg;
  }
  if constexpr ((KINDS & 2) != 0) {
    if (r < per_kg) {
      bwd_dkdv_shared_item<D, kKvDv, SPLIT>(p, tab, lvl * per_kg + r, lds, lds + bwd_kv_buf_bytes<D, kKvDv>());
      return;
    }
    r -= per_kg;
  }
  if constexpr ((KINDS & 4) != 0) bwd_dq_shared_item<D, KW>(p, tab, lvl * KW * per_q + r, lds, lds + bwd_dq_buf_bytes<D>());
}

// ---------------------------------------------------------------------------------------------
// Head-split reduction: dk and dv of key j are the sums over the head splits' partials, added
// in split order (deterministic); dk' is then rotated back by the key's angle, as in the
// kernels' own epilogue.  One thread per (unit, key, column pair c, c + D/2).

template <int D>
__global__ void __launch_bounds__(256) bwd_part_reduce_kernel(BwdParams p, RopeTable tab) {
  const size_t rows = (size_t)p.B * p.Hkv * p.NB * BR;  // (unit, key) rows of the partials
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * (D / 2)) return;
  const int c = (int)(i % (D / 2));
  const size_t row = i / (D / 2);
  const int key = (int)(row % ((size_t)p.NB * BR));
  const size_t unit = row / ((size_t)p.NB * BR);
  if (key >= p.S) return;
  const size_t split = rows * D;  // floats of one split's partials
  const float *pk = p.part + row * D, *pv = p.part + (size_t)p.HS * split + row * D;
  float kx = 0.f, ky = 0.f, vx = 0.f, vy = 0.f;
  for (int hs = 0; hs < p.HS; ++hs) {
    kx += pk[hs * split + c];
    ky += pk[hs * split + c + D / 2];
    vx += pv[hs * split + c];
    vy += pv[hs * split + c + D / 2];
  }
  const float t = turn_fraction(p.k_pos0 + key, tab.rev[c]);
  const float sn = __builtin_amdgcn_sinf(t), cs = __builtin_amdgcn_cosf(t);
  const int g = (int)(unit % p.Hkv), b = (int)(unit / p.Hkv);
  const size_t dst = (((size_t)b * p.S + key) * p.Hkv + g) * D;
  p.dk[dst + rope_src_dim(c, D / 2, tab.interleaved)] = (__bf16)(kx * cs + ky * sn);
  p.dk[dst + rope_src_dim(c + D / 2, D / 2, tab.interleaved)] = (__bf16)(ky * cs - kx * sn);
  p.dv[dst + c] = (__bf16)vx;
  p.dv[dst + c + D / 2] = (__bf16)vy;
}

// dq waves the GPU holds at once (one-wave workgroups), from HIP's occupancy query; cached.
template <int D>
long long bwd_dq_capacity() {
  static long long cap = -1;
  if (cap < 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bwd_dq_kernel<D, false>, 64, 0) != hipSuccess)
      return 0;  // unknown: pairs
    cap = (long long)cus * per_cu;
  }
  return cap;
}

// workgroups of a one-launch kernel the GPU holds at once; cached per head split mode
template <int D, int KINDS>
long long bwd_kv_capacity(bool split) {
  static long long cap[2] = {-1, -1};
  long long &c = cap[split ? 1 : 0];
  if (c < 0) {
    int dev = 0, cus = 0, per_cu = 0;
    const hipError_t e =
        split ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bwd_dkdv_shared_kernel<D, true, KINDS>, 64 * KW, 0)
              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, bwd_dkdv_shared_kernel<D, false, KINDS>, 64 * KW, 0);
    if (e != hipSuccess || hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;  // unknown: two launches
    c = (long long)cus * per_cu;
  }
  return c;
}

template <int D>
hipError_t launch_bwd(const BwdParams &p, const RopeTable &tab, hipStream_t stream) {
  const unsigned kblocks = (unsigned)((long long)p.B * p.Hkv * p.NB);
  const unsigned qblocks = (unsigned)((long long)p.B * p.Hq * p.NB);
  hipLaunchKernelGGL(bwd_prep_kernel<D>, dim3(kblocks + qblocks), dim3(bwd_prep_threads<D>()), 0, stream, p, tab);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if constexpr (D == 256) {
    if ((err = launch_bwd_d256_main(p, tab, stream)) != hipSuccess) return err;
  } else {
    // The per-wave kernels (diagnostics) take work items of single blocks, heaviest first,
    // instead of balanced pairs: for dq when the pairs would leave SIMDs idle, when the key
    // range is long (the waves of one round then sweep nearby key blocks and share them in L2)
    // or when every K/V head serves one query head; for the per-head dk/dv kernel
    // (ATTN_BWD_KV=waves) in that last case only.  (Measured on the workloads: single dq blocks
    // 17% faster on PaLM MQA, 13% on SmolLM MHA, 31% on the 32K shard, 6% slower on
    // Llama-3-8B; single dk/dv blocks 10-19% faster on SmolLM MHA, 5-24% slower on Llama-3-8B
    // and PaLM MQA.)
    bool single_kv = p.G == 1;
    bool single_q = p.G == 1 || p.NB > 64 || (long long)p.B * p.Hq * p.n_pairs < bwd_dq_capacity<D>();
    // diagnostic: ATTN_BWD_ITEMS=pairs or =single forces one kind for every kernel (both give
    // the same bits: each block's sums run in the same order either way)
    if (const char *items = std::getenv("ATTN_BWD_ITEMS")) {
      if (std::strcmp(items, "pairs") == 0) single_kv = single_q = false;
      if (std::strcmp(items, "single") == 0) single_kv = single_q = true;
    }
    const dim3 kv_grid((unsigned)((long long)p.B * p.Hkv * p.HS * (single_kv ? p.NB : p.n_pairs)));
    const dim3 q_grid((unsigned)((long long)p.B * p.Hq * (single_q ? p.NB : p.n_pairs)));
    const dim3 kv_block(64 * p.W);
    // dk/dv: query blocks shared by four consecutive key blocks (default), or (diagnostic,
    // ATTN_BWD_KV=waves) one wave per query head of the group.  (Measured, dk + dv with their
    // head-split reduction, against the per-head kernel with the splits it used alone: 12% less
    // time on Llama-3-8B, 4% on PaLM MQA, 29% on SmolLM MHA, 38% on the 32K shard.)
    // The head splits follow the shared kernel; the per-head one leaves splits past its last
    // pass of heads idle (their partials are zeros).
    bool shared_kv = true;
    if (const char *kvk = std::getenv("ATTN_BWD_KV")) shared_kv = std::strcmp(kvk, "waves") != 0;
    const dim3 skv_grid((unsigned)((long long)p.B * p.Hkv * p.HS * ((p.NB + KW - 1) / KW)));
    auto launch_kv = [&](auto dv, auto split) -> hipError_t {
      constexpr bool DV_ = decltype(dv)::value, SPLIT_ = decltype(split)::value;
      if (shared_kv)
        hipLaunchKernelGGL((bwd_dkdv_shared_kernel<D, SPLIT_, DV_ ? 2 : 1>), skv_grid, dim3(64 * KW), 0, stream, p, tab);
      else if (single_kv)
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, DV_, SPLIT_, true>), kv_grid, kv_block, 0, stream, p, tab);
      else
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, DV_, SPLIT_, false>), kv_grid, kv_block, 0, stream, p, tab);
      return hipGetLastError();
    };
    const std::true_type yes;
    const std::false_type no;
    // dk and dv in one launch when either's work items fit on the GPU at once: each alone would
    // then last as long as its heaviest item, with CUs emptying behind the light ones.  (Measured:
    // dk + dv 25% less time on Llama-3-8B, 31% on PaLM MQA; the same on SmolLM MHA, whose items
    // take two rounds; 11% more on the 32K shard's sixteen rounds, where the two kinds' tiles
    // then share L2.)  ATTN_BWD_KVLAUNCH=split or =one forces the choice (a diagnostic).
    bool one_kv = shared_kv && (long long)skv_grid.x <= bwd_kv_capacity<D, 3>(p.HS > 1);
    if (const char *kvl = std::getenv("ATTN_BWD_KVLAUNCH")) {
      if (std::strcmp(kvl, "split") == 0) one_kv = false;
      if (std::strcmp(kvl, "one") == 0) one_kv = shared_kv;
    }
    bool shared_q = true;
    if (const char *dqk = std::getenv("ATTN_BWD_DQ")) {
      if (std::strcmp(dqk, "shared") == 0) shared_q = true;
      if (std::strcmp(dqk, "regs") == 0) shared_q = false;
    }
    // dq joins that launch when it takes KW heads per workgroup and its items fit at once too
    // (ATTN_BWD_DQLAUNCH=split or =one forces the choice where it can be made, a diagnostic)
    const int passes = (p.G + p.W - 1) / p.W;
    const int qw = p.W == 1 ? bwd_dq_qw<1>() : p.W == 2 ? bwd_dq_qw<2>() : 1;  // query blocks per item
    const long long sq_n = (long long)((p.NB + qw - 1) / qw) * p.B * p.Hkv * passes;
    const bool can_q = one_kv && shared_q && p.W == KW;
    bool one_q = can_q && sq_n <= bwd_kv_capacity<D, 7>(p.HS > 1) &&
                 (long long)skv_grid.x <= bwd_kv_capacity<D, 7>(p.HS > 1);
    if (const char *ql = std::getenv("ATTN_BWD_DQLAUNCH")) {
      if (std::strcmp(ql, "split") == 0) one_q = false;
      if (std::strcmp(ql, "one") == 0) one_q = can_q;
    }
    // head_dim 64: dk and dv from one pass over the query blocks (the probabilities and dS of a
    // step computed once for both products), dq joining that launch when its items fit
    // (ATTN_BWD_KVFUSE=off keeps dk and dv apart, a diagnostic)
    bool fuse_kv = shared_kv && D == 64;
    if (const char *fz = std::getenv("ATTN_BWD_KVFUSE")) fuse_kv = fuse_kv && std::strcmp(fz, "off") != 0;
    if constexpr (D == 64) {
      if (fuse_kv) {
        one_q = shared_q && p.W == KW && sq_n <= bwd_kv_capacity<D, 12>(p.HS > 1) &&
                (long long)skv_grid.x <= bwd_kv_capacity<D, 12>(p.HS > 1);
        if (const char *ql = std::getenv("ATTN_BWD_DQLAUNCH")) {
          if (std::strcmp(ql, "split") == 0) one_q = false;
          if (std::strcmp(ql, "one") == 0) one_q = shared_q && p.W == KW;
        }
        const dim3 grid2((unsigned)(skv_grid.x + (one_q ? sq_n : 0)));
        if (one_q && p.HS > 1)
          hipLaunchKernelGGL((bwd_dkdv_shared_kernel<D, true, 12>), grid2, dim3(64 * KW), 0, stream, p, tab);
        else if (one_q)
          hipLaunchKernelGGL((bwd_dkdv_shared_kernel<D, false, 12>), grid2, dim3(64 * KW), 0, stream, p, tab);
        else if (p.HS > 1)
          hipLaunchKernelGGL((bwd_dkdv_shared_kernel<D, true, 8>), grid2, dim3(64 * KW), 0, stream, p, tab);
        else
          hipLaunchKernelGGL((bwd_dkdv_shared_kernel<D, false, 8>), grid2, dim3(64 * KW), 0, stream, p, tab);
        if ((err = hipGetLastError()) != hipSuccess) return err;
      }
    }
    if (fuse_kv) {
      // (launched above)
    } else if (one_kv) {
      const dim3 grid2((unsigned)(2LL * skv_grid.x + (one_q ? sq_n : 0)));
      if (one_q && p.HS > 1)
        hipLaunchKernelGGL((bwd_dkdv_shared_kernel<D, true, 7>), grid2, dim3(64 * KW), 0, stream, p, tab);
      else if (one_q)
        hipLaunchKernelGGL((bwd_dkdv_shared_kernel<D, false, 7>), grid2, dim3(64 * KW), 0, stream, p, tab);
      else if (p.HS > 1)
        hipLaunchKernelGGL((bwd_dkdv_shared_kernel<D, true, 3>), grid2, dim3(64 * KW), 0, stream, p, tab);
      else
        hipLaunchKernelGGL((bwd_dkdv_shared_kernel<D, false, 3>), grid2, dim3(64 * KW), 0, stream, p, tab);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    } else if (p.HS > 1) {
      if ((err = launch_kv(yes, yes)) != hipSuccess) return err;  // dv
      if ((err = launch_kv(no, yes)) != hipSuccess) return err;   // dk
    } else {
      if ((err = launch_kv(yes, no)) != hipSuccess) return err;
      if ((err = launch_kv(no, no)) != hipSuccess) return err;
    }
    if (one_q) {
      // (dq ran in the launch above)
    } else if (shared_q) {
      const dim3 sq_grid((unsigned)sq_n);
      switch (p.W) {
        case 1: hipLaunchKernelGGL((bwd_dq_shared_kernel<D, 1>), sq_grid, dim3(256), 0, stream, p, tab); break;
        case 2: hipLaunchKernelGGL((bwd_dq_shared_kernel<D, 2>), sq_grid, dim3(256), 0, stream, p, tab); break;
        case 3: hipLaunchKernelGGL((bwd_dq_shared_kernel<D, 3>), sq_grid, dim3(192), 0, stream, p, tab); break;
        default: hipLaunchKernelGGL((bwd_dq_shared_kernel<D, 4>), sq_grid, dim3(256), 0, stream, p, tab); break;
      }
    } else if (single_q) {
      hipLaunchKernelGGL((bwd_dq_kernel<D, true>), q_grid, dim3(64), 0, stream, p, tab);
    } else {
      hipLaunchKernelGGL((bwd_dq_kernel<D, false>), q_grid, dim3(64), 0, stream, p, tab);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (p.HS > 1) {
    const long long n = (long long)p.B * p.Hkv * p.NB * BR * (D / 2);
    hipLaunchKernelGGL(bwd_part_reduce_kernel<D>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, tab);
    return hipGetLastError();
  }
  return hipSuccess;
}

template hipError_t launch_bwd<64>(const BwdParams &, const RopeTable &, hipStream_t);
template hipError_t launch_bwd<128>(const BwdParams &, const RopeTable &, hipStream_t);
template hipError_t launch_bwd<256>(const BwdParams &, const RopeTable &, hipStream_t);

}  // namespace attn
