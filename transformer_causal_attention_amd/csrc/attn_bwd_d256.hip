// Backward of the fused causal RoPE-GQA attention at head_dim 256 (the PaLM page's 540B head
// size, section 3): the dk/dv and dq kernels.  The layout passes, the head-split reduction and
// the arithmetic they share with the other head sizes are in attn_bwd.hip.

#include "attn_bwd_common.h"

namespace attn {

// The head_dim 64 and 128 kernels keep a block's operands in registers: at 256 dims the dk
// kernel would need ~650 VGPRs.  Here the block that stays fixed over a kernel's loop lives in
// LDS (the key block's rotated keys and values for dk/dv, the query block's rotated queries and
// dout for dq), every MFMA operand of it is one 16-byte LDS read, and the moving block's
// operands are read from the prepared tiles per step.  Same arithmetic, operand layouts,
// visibility and masks as the head_dim 64 and 128 kernels.

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
    const bool key_ok_all = (kb + 1) * BR <= p.S;  // every key of the block is a real one
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

hipError_t launch_bwd_d256_main(const BwdParams &p, const RopeTable &tab, dim3 kv_grid, dim3 q_grid,
                                hipStream_t stream) {
  if (p.HS > 1) {
    hipLaunchKernelGGL((bwd_dkdv_d256_kernel<true, true>), kv_grid, dim3(64 * p.W), 0, stream, p, tab);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((bwd_dkdv_d256_kernel<false, true>), kv_grid, dim3(64 * p.W), 0, stream, p, tab);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_d256_kernel<true, false>), kv_grid, dim3(64 * p.W), 0, stream, p, tab);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((bwd_dkdv_d256_kernel<false, false>), kv_grid, dim3(64 * p.W), 0, stream, p, tab);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(bwd_dq_d256_kernel, q_grid, dim3(64), 0, stream, p, tab);
  return hipGetLastError();
}

}  // namespace attn
