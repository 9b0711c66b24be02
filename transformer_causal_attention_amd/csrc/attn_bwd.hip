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
// Five launches, 32-row blocks of queries and keys throughout:
//   bwd_prep_k  rotated keys in "c" and "t" layouts, values in "c" layout, per key block;
//   bwd_prep_q  rotated queries (scaled) in "c" and "t" layouts, dout in both, and per row
//               lse * log2(e) and rowsum(dout * out), per query block;
//   bwd_dkdv    twice, for dv and for dk: one workgroup per (b, K/V head, pair of key blocks
//               kb, NB-1-kb), one wave per query head of the group (up to 4, each looping over
//               the rest): for every query block that sees the key block, S = Q K^T (and
//               dP = dO V^T) on MFMA with one key per lane, then dv += P^T dO or
//               dk += dS^T Q; the waves' sums are added through LDS, dk is rotated back, and
//               each row is written once (no atomics);
//   bwd_dq      one wave per (b, query head, pair of query blocks): S^T = K Q^T and
//               dP^T = V dO^T with one query per lane, dq += dS K; rotated back and written.
// A call may be one block of a longer sequence (one step of ring attention's backward): queries
// at positions q_pos0 + i, keys at k_pos0 + j, key j visible to query i iff j <= i + delta with
// delta = q_pos0 - k_pos0; out and lse are then the forward's results over every key block, and
// dq (dk, dv) is this key block's (query block's) part of the gradient.  Block kb of keys is seen
// by query blocks from qb_lo(kb) on, query block qb sees key blocks below kb_end(qb), and a
// block pair needs the element mask only where some key is later than some row.
// Causal work is balanced by pairing block kb with NB-1-kb.  Operands are read straight from
// the pre-laid-out tiles into registers (16-byte loads, each a whole MFMA operand per lane), so
// no LDS is needed outside the dk/dv reduction and the layout passes.
//
// MFMA v_mfma_f32_32x32x16_bf16: A lane l holds row l%32, k = 8(l/32) .. +7; B lane l holds
// column l%32, same k; the result's register v in lane l is row 8(v/4) + 4(l/32) + v%4,
// column l%32.  A score result packed as bf16 (registers 8t .. 8t+7 -> one operand) therefore
// lists its rows in the order 16t + swap23(8(l/32) + e), which is the row order of the "t"
// layout.

#include "attn_device.h"

namespace attn {

namespace {

constexpr int BR = 32;  // rows per block

__device__ __forceinline__ f32x16 bwd_mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Workgroup i runs on XCD i % 8 (round-robin dispatch).  This renumbers the n workgroups so
// that each XCD gets a contiguous run of the logical order, i.e. the blocks of the same K/V
// head group, whose tiles then stay in that XCD's L2.  A bijection on [0, n) for any n.
__device__ __forceinline__ int xcd_order(int i, int n) {
  const int x = i & 7, q = n >> 3, r = n & 7;
  return x * q + min(x, r) + (i >> 3);
}

__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// floor(a / b) for b > 0 and any sign of a
__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

__device__ __forceinline__ bf16x8 ld16(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// 16 bytes at byte voff (per lane) + soff (uniform) of a buffer: the base stays in scalar
// registers and each lane keeps one 32-bit offset, not a 64-bit address per operand stream.
// Constant parts of an offset go into soff, so that no lane holds a register per operand.
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

// Row of result register v in lane half hh.
__device__ __forceinline__ int res_row(int v, int hh) { return 8 * (v >> 2) + 4 * hh + (v & 3); }

// Writes a 32-row block staged in LDS (rows of stride LS elements) in "t" layout: 4*D chunks of
// 16 bytes, chunk (half, j, column) = rows 16 half + swap23(8 j + e), e = 0..7, of that column.
template <int D, int LS>
__device__ __forceinline__ void write_t_layout(const uint16_t *lds, __bf16 *dst, int tid, int nthreads) {
  for (int ch = tid; ch < 4 * D; ch += nthreads) {
    const int col = ch % D;
    const int hj = ch / D;  // 2 half + j
    const int half = hj >> 1, j = hj & 1;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int r0 = 16 * half + swap23(8 * j + e);
      const int r1 = 16 * half + swap23(8 * j + e + 1);
      w[e / 2] = (uint32_t)lds[r0 * LS + col] | ((uint32_t)lds[r1 * LS + col] << 16);
    }
    *reinterpret_cast<u32x4 *>(dst + (size_t)ch * 8) = w;
  }
}

// Rotation of 8 pairs (x_i, y_i) = (dims 8c + i, D/2 + 8c + i) of one row at position pos.
template <int D>
__device__ __forceinline__ void rotate8(const RopeTable &tab, int c, int pos, const u32x4 &xr, const u32x4 &yr,
                                        float x[8], float y[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t xw = xr[i / 2], yw = yr[i / 2];
    const float xv = (i & 1) ? bf16_hi(xw) : bf16_lo(xw);
    const float yv = (i & 1) ? bf16_hi(yw) : bf16_lo(yw);
    const float t = turn_fraction(pos, tab.rev[8 * c + i]);
    const float sn = __builtin_amdgcn_sinf(t), cs = __builtin_amdgcn_cosf(t);
    x[i] = xv * cs - yv * sn;
    y[i] = yv * cs + xv * sn;
  }
}

__device__ __forceinline__ u32x4 pack8(const float a[8], float s) {
  return u32x4{pack_bf16x2(a[0] * s, a[1] * s), pack_bf16x2(a[2] * s, a[3] * s), pack_bf16x2(a[4] * s, a[5] * s),
               pack_bf16x2(a[6] * s, a[7] * s)};
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// Layout passes.  256 threads; item = row * NCH + c covers dims 8c .. 8c+7 and D/2 + 8c .. of
// one row (NCH = D/16 pairs of 8-dim chunks).

template <int D>
__global__ void __launch_bounds__(256) bwd_prep_k_kernel(BwdParams p, RopeTable tab) {
  constexpr int NCH = D / 16;
  constexpr int LS = D + 8;
  constexpr int T = BR * D;  // elements per tile
  __shared__ __attribute__((aligned(16))) uint16_t sk[BR * LS];
  const int tid = threadIdx.x;
  const int kb = blockIdx.x % p.NB;
  const int unit = blockIdx.x / p.NB;  // b * Hkv + g
  const int g = unit % p.Hkv, b = unit / p.Hkv;
  const size_t tile = (size_t)blockIdx.x * T;
  for (int item = tid; item < BR * NCH; item += 256) {  // one pass, two at head_dim 256
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
  write_t_layout<D, LS>(sk, p.kt + tile, tid, 256);
}

template <int D>
__global__ void __launch_bounds__(256) bwd_prep_q_kernel(BwdParams p, RopeTable tab) {
  constexpr int NCH = D / 16;
  constexpr int LS = D + 8;
  constexpr int T = BR * D;
  __shared__ __attribute__((aligned(16))) uint16_t sq[BR * LS];
  __shared__ __attribute__((aligned(16))) uint16_t sd[BR * LS];
  const int tid = threadIdx.x;
  const int qb = blockIdx.x % p.NB;
  const int unit = blockIdx.x / p.NB;  // b * Hq + h
  const int h = unit % p.Hq, b = unit / p.Hq;
  const size_t tile = (size_t)blockIdx.x * T;
  // one pass, two at head_dim 256 (the NCH items of a row are consecutive lanes of one wave in
  // either pass, for the row sums below)
  for (int item = tid; item < BR * NCH; item += 256) {
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
  write_t_layout<D, LS>(sq, p.qt + tile, tid, 256);
  write_t_layout<D, LS>(sd, p.dt + tile, tid, 256);
}

// ---------------------------------------------------------------------------------------------
// dv (DV) or dk (!DV).  Workgroup: (b, g, key-block pair), W waves; wave w takes the group's
// heads w, w+W, ...  The two gradients are separate kernels so that each holds one set of
// accumulators and has the registers to load the next query block's operands while it uses the
// current ones; the dv kernel needs neither dP nor dout in "c" layout.

template <int D, bool DV, bool SPLIT>
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
  const int blk = xcd_order(blockIdx.x, gridDim.x);
  const int pair = blk % p.n_pairs;
  const int n_hs = SPLIT ? p.HS : 1;          // head splits (SPLIT: more than one)
  const int hs = SPLIT ? (blk / p.n_pairs) % n_hs : 0;
  const int unit = blk / p.n_pairs / n_hs;     // b * Hkv + g
  const int g = unit % p.Hkv, b = unit / p.Hkv;
  const int c_off = hh * BR * 8 + l32 * 8;  // this lane's operand in a "c" tile (chunk 2kk + hh)

#pragma unroll 1
  for (int side = 0; side < 2; ++side) {
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
    f32x16 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};

    // query-block operands, two sets (see the dq kernel)
    bf16x8 qa[2][NKK], da[2][NKK], tb[2][2][NCB];
    f32x4 L[2][4], Dd[2][4];
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
      auto load_q = [&](int qb, int buf) __attribute__((always_inline)) {
        const uint32_t st = (uint32_t)qb * T * 2, sr = (uint32_t)qb * BR * 4;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          qa[buf][kk] = __builtin_bit_cast(bf16x8, bld16(qbuf, v_c, st + kk * 2 * BR * 16));
          if (!DV) da[buf][kk] = __builtin_bit_cast(bf16x8, bld16(dbuf, v_c, st + kk * 2 * BR * 16));
        }
        // per-row lse and rowsum for this lane's rows 8c + 4hh + 0..3
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          L[buf][c] = __builtin_bit_cast(f32x4, bld16(lbuf, v_r, sr + 32 * c));
          if (!DV) Dd[buf][c] = __builtin_bit_cast(f32x4, bld16(ddbuf, v_r, sr + 32 * c));
        }
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            tb[buf][tt][cb] = __builtin_bit_cast(bf16x8, bld16(tbuf, v_t, st + (tt * 2 * D + 32 * cb) * 16));
      };
      auto step = [&](int qb, int buf) __attribute__((always_inline)) {
        f32x16 s = f32x16{}, dp = f32x16{};
        // (the LDS index goes through an empty asm so that the reads stay in the step)
        int ki = lane;
        if (DV) asm volatile("" : "+v"(ki));
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          s = bwd_mfma(qa[buf][kk], DV ? kl[64 * kk + ki] : kf[kk], s);
          if (!DV) dp = bwd_mfma(da[buf][kk], vf[kk], dp);
        }
        // key kb*32 + l32 is later than row qb*32 + r iff l32 - r > rel, i.e. (r = res_row(v, hh))
        // iff 8(v/4) + v%4 < thr.  One threshold per lane and step, compared with constants and
        // applied by selects: a key past S masks every row (thr 32), a block pair with no later
        // key none (thr 0).  (A short-circuit test here becomes a branch around each exp, and
        // per-lane constants per v would stay live across the loop.)
        const int rel = BR * (qb - kb) + delta;
        const int thr = !key_ok ? 32 : (p.causal && rel < BR - 1) ? l32 - 4 * hh - rel : 0;
        bf16x8 op[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          u32x4 wv;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float x[2];
#pragma unroll
            for (int z = 0; z < 2; ++z) {
              const int v = 8 * tt + e + z;
              float pr = __builtin_amdgcn_exp2f(s[v] - L[buf][v >> 2][v & 3]);
              pr = 8 * (v >> 2) + (v & 3) < thr ? 0.f : pr;
              x[z] = DV ? pr : pr * (dp[v] - Dd[buf][v >> 2][v & 3]);
            }
            wv[e / 2] = pack_bf16x2(x[0], x[1]);
          }
          op[tt] = __builtin_bit_cast(bf16x8, wv);
        }
        // dv += P^T dO, dk += dS^T (q'/sqrt(D))
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) acc[cb] = bwd_mfma(op[tt], tb[buf][tt][cb], acc[cb]);
      };
      // from the last query block down, so that the workgroups of a group sweep the same
      // query tiles at about the same time; the clamped index re-reads the last block
      load_q(p.NB - 1, 0);
      for (int qb = p.NB - 1; qb >= qb_lo; qb -= 2) {
        load_q(max(qb - 1, qb_lo), 1);
        step(qb, 0);
        if (qb - 1 >= qb_lo) {
          load_q(max(qb - 2, qb_lo), 0);
          step(qb - 1, 1);
        }
      }
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
// dq.  One wave per (b, h, query-block pair).

template <int D>
__global__ void __launch_bounds__(64, D == 64 ? 2 : 1) bwd_dq_kernel(BwdParams p, RopeTable tab) {
  constexpr int NKK = D / 16;
  constexpr int NCB = D / 32;
  constexpr int T = BR * D;
  const int lane = threadIdx.x;
  const int l32 = lane & 31, hh = lane >> 5;
  const int blk = xcd_order(blockIdx.x, gridDim.x);
  const int pair = blk % p.n_pairs;
  const int qunit = blk / p.n_pairs;  // b * Hq + h
  const int h = qunit % p.Hq, b = qunit / p.Hq;
  const int g = h / p.G;
  const size_t kunit = (size_t)b * p.Hkv + g;
  const int c_off = hh * BR * 8 + l32 * 8;

  for (int side = 0; side < 2; ++side) {
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
    // key-block operands, two sets: the next block's are loaded while the current one is used
    // (the index is clamped, so the last step re-reads its own block instead of branching)
    bf16x8 ka[2][NKK], va[2][NKK], kt[2][2][NCB];
    // this K/V head's run of key blocks as buffers (NB * T * 2 < 2^31 bytes), per-lane byte offsets
    const uint32_t run_t = (uint32_t)p.NB * T * 2;
    const __amdgpu_buffer_rsrc_t kbuf = raw_buffer(p.kc + kunit * p.NB * T, run_t);
    const __amdgpu_buffer_rsrc_t vbuf = raw_buffer(p.vc + kunit * p.NB * T, run_t);
    const __amdgpu_buffer_rsrc_t tbuf = raw_buffer(p.kt + kunit * p.NB * T, run_t);
    const uint32_t v_c = 2u * c_off, v_t = 16u * (hh * D + l32);
    auto load_kv = [&](int kb, int buf) __attribute__((always_inline)) {
      const uint32_t st = (uint32_t)kb * T * 2;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        ka[buf][kk] = __builtin_bit_cast(bf16x8, bld16(kbuf, v_c, st + kk * 2 * BR * 16));
        va[buf][kk] = __builtin_bit_cast(bf16x8, bld16(vbuf, v_c, st + kk * 2 * BR * 16));
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          kt[buf][tt][cb] = __builtin_bit_cast(bf16x8, bld16(tbuf, v_t, st + (tt * 2 * D + 32 * cb) * 16));
    };
    auto step = [&](int kb, int buf) __attribute__((always_inline)) {
      f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        st = bwd_mfma(ka[buf][kk], qf[kk], st);
        dpt = bwd_mfma(va[buf][kk], df[kk], dpt);
      }
      // key kb*32 + k is later than row qb*32 + l32 iff k - l32 > rel, i.e. (k = res_row(v, hh))
      // iff 8(v/4) + v%4 > thr: one threshold per lane and step against constants, applied by
      // selects (thr 27 masks nothing).  Keys past S: those of the last block from S - 32 kb on.
      const int rel = BR * (qb - kb) + delta;
      const int thr = (p.causal && rel < BR - 1) ? rel + l32 - 4 * hh : 27;
      const int kend = p.S - kb * BR - 4 * hh;  // key 8(v/4) + v%4 + 4hh < S iff 8(v/4) + v%4 < kend
      bf16x8 sa[2];
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
            pr = ((8 * (v >> 2) + (v & 3) > thr) | (8 * (v >> 2) + (v & 3) >= kend)) ? 0.f : pr;
            sv[z] = pr * (dpt[v] - Dq);
          }
          ws[e / 2] = pack_bf16x2(sv[0], sv[1]);
        }
        sa[tt] = __builtin_bit_cast(bf16x8, ws);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) dq[cb] = bwd_mfma(sa[tt], kt[buf][tt][cb], dq[cb]);
    };
    load_kv(0, 0);
    for (int kb = 0; kb < kb_end; kb += 2) {
      load_kv(min(kb + 1, kb_end - 1), 1);
      step(kb, 0);
      if (kb + 1 < kb_end) {
        load_kv(min(kb + 2, kb_end - 1), 0);
        step(kb + 1, 1);
      }
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
// head_dim 256 (the PaLM page's 540B head size, section 3).  The kernels above keep a block's
// operands in registers: at 256 dims the dk kernel would need ~650 VGPRs.  Here the block that
// stays fixed over a kernel's loop lives in LDS (the key block's rotated keys and values for
// dk/dv, the query block's rotated queries and dout for dq), every MFMA operand of it is one
// 16-byte LDS read, and the moving block's operands are read from the prepared tiles per step.
// Same arithmetic, operand layouts, visibility and masks as the kernels above.

__device__ __forceinline__ bf16x8 lds16(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

template <bool DV, bool SPLIT>
__global__ void __launch_bounds__(256, 1) bwd_dkdv_d256_kernel(BwdParams p, RopeTable tab) {
  constexpr int D = 256;
  constexpr int NKK = D / 16;
  constexpr int NCB = D / 32;
  constexpr int T = BR * D;
  constexpr int RED = NCB * 16 * 64;
  __shared__ float red[3][RED];
  __shared__ __attribute__((aligned(16))) __bf16 kv[DV ? 1 : 2][T];  // key block: rotated keys, values
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int nthreads = 64 * p.W;
  const int l32 = lane & 31, hh = lane >> 5;
  const int blk = xcd_order(blockIdx.x, gridDim.x);
  const int pair = blk % p.n_pairs;
  const int n_hs = SPLIT ? p.HS : 1;          // head splits (SPLIT: more than one)
  const int hs = SPLIT ? (blk / p.n_pairs) % n_hs : 0;
  const int unit = blk / p.n_pairs / n_hs;     // b * Hkv + g
  const int g = unit % p.Hkv, b = unit / p.Hkv;
  const int c_off = hh * BR * 8 + l32 * 8;  // this lane's operand in a "c" tile (chunk 2kk + hh)
  const int delta = p.q_pos0 - p.k_pos0;

  for (int side = 0; side < 2; ++side) {
    const int kb = side == 0 ? pair : p.NB - 1 - pair;
    if (side == 1 && kb == pair) break;
    const size_t ktile = ((size_t)unit * p.NB + kb) * T;
    __syncthreads();  // the previous block's operands are no longer read
    for (int i = threadIdx.x; i < T / 8; i += nthreads) {
      *reinterpret_cast<u32x4 *>(&kv[0][8 * i]) = *reinterpret_cast<const u32x4 *>(p.kc + ktile + 8 * i);
      if (!DV) *reinterpret_cast<u32x4 *>(&kv[DV ? 0 : 1][8 * i]) = *reinterpret_cast<const u32x4 *>(p.vc + ktile + 8 * i);
    }
    __syncthreads();
    const bool key_ok = kb * BR + l32 < p.S;
    f32x16 acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};
    const int qb_lo = p.causal ? max(0, floor_div(BR * kb - delta, BR)) : 0;
    for (int hc = wave + hs * p.W; hc < p.G; hc += p.W * n_hs) {
      const size_t qunit = (size_t)b * p.Hq + g * p.G + hc;
      for (int qb = p.NB - 1; qb >= qb_lo; --qb) {
        const size_t qtile = (qunit * p.NB + qb) * T;
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          sc = bwd_mfma(ld16(p.qc + qtile + c_off + kk * 2 * BR * 8), lds16(&kv[0][c_off + kk * 2 * BR * 8]), sc);
          if (!DV)
            dp = bwd_mfma(ld16(p.dc + qtile + c_off + kk * 2 * BR * 8), lds16(&kv[DV ? 0 : 1][c_off + kk * 2 * BR * 8]),
                          dp);
        }
        // per-row lse and rowsum for this lane's rows 8c + 4hh + 0..3
        const size_t r0 = (qunit * p.NB + qb) * BR + 4 * hh;
        f32x4 L[4], Dd[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          L[c] = *reinterpret_cast<const f32x4 *>(p.l2 + r0 + 8 * c);
          Dd[c] = DV ? f32x4{} : *reinterpret_cast<const f32x4 *>(p.dd + r0 + 8 * c);
        }
        // key kb*32 + l32 is later than row qb*32 + r iff l32 - r > rel, i.e. (r = res_row(v, hh))
        // iff 8(v/4) + v%4 < thr.  One threshold per lane and step, compared with constants and
        // applied by selects: a key past S masks every row (thr 32), a block pair with no later
        // key none (thr 0).  (A short-circuit test here becomes a branch around each exp, and
        // per-lane constants per v would stay live across the loop.)
        const int rel = BR * (qb - kb) + delta;
        const int thr = !key_ok ? 32 : (p.causal && rel < BR - 1) ? l32 - 4 * hh - rel : 0;
        bf16x8 op[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          u32x4 wv;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float x[2];
#pragma unroll
            for (int z = 0; z < 2; ++z) {
              const int v = 8 * tt + e + z;
              float pr = __builtin_amdgcn_exp2f(sc[v] - L[v >> 2][v & 3]);
              pr = 8 * (v >> 2) + (v & 3) < thr ? 0.f : pr;
              x[z] = DV ? pr : pr * (dp[v] - Dd[v >> 2][v & 3]);
            }
            wv[e / 2] = pack_bf16x2(x[0], x[1]);
          }
          op[tt] = __builtin_bit_cast(bf16x8, wv);
        }
        // dv += P^T dO, dk += dS^T (q'/sqrt(D))
        const __bf16 *tsrc = DV ? p.dt : p.qt;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            acc[cb] = bwd_mfma(op[tt], ld16(tsrc + qtile + ((size_t)(tt * 2 + hh) * D + 32 * cb + l32) * 8), acc[cb]);
      }
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
          const int il = DV ? 0 : tab.interleaved;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) dst0[dst + rope_src_dim(32 * cb + l32, D / 2, il)] = (__bf16)acc[cb][v];
        }
      }
      }
    }
  }
}

__global__ void __launch_bounds__(64, 1) bwd_dq_d256_kernel(BwdParams p, RopeTable tab) {
  constexpr int D = 256;
  constexpr int NKK = D / 16;
  constexpr int NCB = D / 32;
  constexpr int T = BR * D;
  __shared__ __attribute__((aligned(16))) __bf16 qd[2][T];  // query block: scaled rotated queries, dout
  const int lane = threadIdx.x;
  const int l32 = lane & 31, hh = lane >> 5;
  const int blk = xcd_order(blockIdx.x, gridDim.x);
  const int pair = blk % p.n_pairs;
  const int qunit = blk / p.n_pairs;  // b * Hq + h
  const int h = qunit % p.Hq, b = qunit / p.Hq;
  const int g = h / p.G;
  const size_t kunit = (size_t)b * p.Hkv + g;
  const int c_off = hh * BR * 8 + l32 * 8;
  const int delta = p.q_pos0 - p.k_pos0;

  for (int side = 0; side < 2; ++side) {
    const int qb = side == 0 ? pair : p.NB - 1 - pair;
    if (side == 1 && qb == pair) break;
    const size_t qtile = ((size_t)qunit * p.NB + qb) * T;
    __syncthreads();  // the previous block's operands are no longer read
    for (int i = lane; i < T / 8; i += 64) {
      *reinterpret_cast<u32x4 *>(&qd[0][8 * i]) = *reinterpret_cast<const u32x4 *>(p.qc + qtile + 8 * i);
      *reinterpret_cast<u32x4 *>(&qd[1][8 * i]) = *reinterpret_cast<const u32x4 *>(p.dc + qtile + 8 * i);
    }
    __syncthreads();
    // this lane's query: row l32 of the block
    const float Lq = p.l2[((size_t)qunit * p.NB + qb) * BR + l32];
    const float Dq = p.dd[((size_t)qunit * p.NB + qb) * BR + l32];
    f32x16 dq[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) dq[cb] = f32x16{};
    const int kb_end = p.causal ? min(p.NB, max(0, floor_div(BR * qb + BR - 1 + delta, BR) + 1)) : p.NB;
    for (int kb = 0; kb < kb_end; ++kb) {
      const size_t ktile = (kunit * p.NB + kb) * T;
      f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        st = bwd_mfma(ld16(p.kc + ktile + c_off + kk * 2 * BR * 8), lds16(&qd[0][c_off + kk * 2 * BR * 8]), st);
        dpt = bwd_mfma(ld16(p.vc + ktile + c_off + kk * 2 * BR * 8), lds16(&qd[1][c_off + kk * 2 * BR * 8]), dpt);
      }
      // key kb*32 + k is later than row qb*32 + l32 iff k - l32 > rel, i.e. (k = res_row(v, hh))
      // iff 8(v/4) + v%4 > thr: one threshold per lane and step against constants, applied by
      // selects (thr 27 masks nothing).  Keys past S: those of the last block from S - 32 kb on.
      const int rel = BR * (qb - kb) + delta;
      const int thr = (p.causal && rel < BR - 1) ? rel + l32 - 4 * hh : 27;
      const int kend = p.S - kb * BR - 4 * hh;  // key 8(v/4) + v%4 + 4hh < S iff 8(v/4) + v%4 < kend
      bf16x8 sa[2];
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
            pr = ((8 * (v >> 2) + (v & 3) > thr) | (8 * (v >> 2) + (v & 3) >= kend)) ? 0.f : pr;
            sv[z] = pr * (dpt[v] - Dq);
          }
          ws[e / 2] = pack_bf16x2(sv[0], sv[1]);
        }
        sa[tt] = __builtin_bit_cast(bf16x8, ws);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          dq[cb] = bwd_mfma(sa[tt], ld16(p.kt + ktile + ((size_t)(tt * 2 + hh) * D + 32 * cb + l32) * 8), dq[cb]);
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

template <int D>
hipError_t launch_bwd(const BwdParams &p, const RopeTable &tab, hipStream_t stream) {
  const unsigned kblocks = (unsigned)((long long)p.B * p.Hkv * p.NB);
  const unsigned qblocks = (unsigned)((long long)p.B * p.Hq * p.NB);
  hipLaunchKernelGGL(bwd_prep_k_kernel<D>, dim3(kblocks), dim3(256), 0, stream, p, tab);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(bwd_prep_q_kernel<D>, dim3(qblocks), dim3(256), 0, stream, p, tab);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const dim3 kv_grid((unsigned)((long long)p.B * p.Hkv * p.n_pairs * p.HS));
  const dim3 q_grid((unsigned)((long long)p.B * p.Hq * p.n_pairs));
  if constexpr (D == 256) {
    if (p.HS > 1) {
      hipLaunchKernelGGL((bwd_dkdv_d256_kernel<true, true>), kv_grid, dim3(64 * p.W), 0, stream, p, tab);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      hipLaunchKernelGGL((bwd_dkdv_d256_kernel<false, true>), kv_grid, dim3(64 * p.W), 0, stream, p, tab);
    } else {
      hipLaunchKernelGGL((bwd_dkdv_d256_kernel<true, false>), kv_grid, dim3(64 * p.W), 0, stream, p, tab);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      hipLaunchKernelGGL((bwd_dkdv_d256_kernel<false, false>), kv_grid, dim3(64 * p.W), 0, stream, p, tab);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(bwd_dq_d256_kernel, q_grid, dim3(64), 0, stream, p, tab);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  } else {
    if (p.HS > 1) {
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, true>), kv_grid, dim3(64 * p.W), 0, stream, p, tab);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, true>), kv_grid, dim3(64 * p.W), 0, stream, p, tab);
    } else {
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, false>), kv_grid, dim3(64 * p.W), 0, stream, p, tab);
      if ((err = hipGetLastError()) != hipSuccess) return err;
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, false>), kv_grid, dim3(64 * p.W), 0, stream, p, tab);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(bwd_dq_kernel<D>, q_grid, dim3(64), 0, stream, p, tab);
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
