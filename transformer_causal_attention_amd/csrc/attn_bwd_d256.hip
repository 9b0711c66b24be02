// Backward of the fused causal RoPE-GQA attention at head_dim 256 (the PaLM page's 540B head
// size, section 3): the dk/dv and dq kernels.  The layout passes, the head-split reduction and
// the arithmetic they share with the other head sizes are in attn_bwd.hip.

#include "attn_bwd_common.h"

namespace attn {

// The head_dim 64 and 128 kernels keep a block's operands in registers: at 256 dims the dk
// kernel would need ~650 VGPRs.  Here the block that stays fixed over a kernel's loop lives in
// LDS (the key block's rotated keys and values for dk/dv, the query block's rotated queries and
// dout for dq), every MFMA operand of it is one 16-byte LDS read, and the moving block's
// operands are read from the prepared tiles through buffer resources, each register reloaded
// with the next block's operand as soon as its MFMA has read it (the dk/dv kernel's operands of
// the gradient product, which would not fit beside them, are loaded at the start of the step
// that uses them).  Same arithmetic, operand layouts, visibility and masks as the head_dim 64
// and 128 kernels.

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
  // One key block per workgroup, the heaviest first: a causal key block kb is seen by the
  // NB - kb query blocks from kb on, so the grid's rounds run from kb = 0 up and the last,
  // partial round holds the lightest blocks.
  const int n_hs = SPLIT ? p.HS : 1;          // head splits (SPLIT: more than one)
  const int per_kb = p.B * p.Hkv * n_hs;
  const int kb_rank = blockIdx.x / per_kb, rest = blockIdx.x % per_kb;
  const int hs = SPLIT ? rest % n_hs : 0;
  const int unit = rest / n_hs;                // b * Hkv + g
  const int g = unit % p.Hkv, b = unit / p.Hkv;
  const int c_off = hh * BR * 8 + l32 * 8;  // this lane's operand in a "c" tile (chunk 2kk + hh)
  const int delta = p.q_pos0 - p.k_pos0;

  {
    const int kb = kb_rank;
    const size_t ktile = ((size_t)unit * p.NB + kb) * T;
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
    const __bf16 *tsrc = DV ? p.dt : p.qt;
    for (int hc = wave + hs * p.W; hc < p.G; hc += p.W * n_hs) {
      const size_t qunit = (size_t)b * p.Hq + g * p.G + hc;
      // the moving query block's operands, one register set: each register is reloaded with the
      // next block's operand as soon as its MFMA has read it
      bf16x8 qa[NKK], da[DV ? 1 : NKK], tb[2][NCB];
      f32x4 L[4], Dd[4];
      // this head's run of query blocks as buffers (NB * T * 2 < 2^31 bytes): a base in scalar
      // registers and one 32-bit offset per lane, not a 64-bit address per operand
      const uint32_t run_t = (uint32_t)p.NB * T * 2, run_r = (uint32_t)p.NB * BR * 4;
      const __amdgpu_buffer_rsrc_t qbuf = raw_buffer(p.qc + qunit * p.NB * T, run_t);
      const __amdgpu_buffer_rsrc_t dbuf = raw_buffer(p.dc + qunit * p.NB * T, run_t);
      const __amdgpu_buffer_rsrc_t tbuf = raw_buffer(tsrc + qunit * p.NB * T, run_t);
      const __amdgpu_buffer_rsrc_t lbuf = raw_buffer(p.l2 + qunit * p.NB * BR, run_r);
      const __amdgpu_buffer_rsrc_t ddbuf = raw_buffer(p.dd + qunit * p.NB * BR, run_r);
      const uint32_t v_c = 2u * c_off, v_t = 16u * (hh * D + l32), v_r = 16u * hh;
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
      // key kb*32 + l32 is later than row qb*32 + r iff l32 - r > rel, i.e. (r = res_row(v, hh))
      // iff 8(v/4) + v%4 < thr: one threshold per lane and step, compared with constants and
      // applied by selects, only in the steps that need it (a key past S masks every row)
      auto probs = [&](const f32x16 &sc, const f32x16 &dp, bool masked, int thr, bf16x8 (&op)[2])
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
              float pr = __builtin_amdgcn_exp2f(sc[v] - L[v >> 2][v & 3]);
              if (masked) pr = 8 * (v >> 2) + (v & 3) < thr ? 0.f : pr;
              x[z] = DV ? pr : pr * (dp[v] - Dd[v >> 2][v & 3]);
            }
            wv[e / 2] = pack_bf16x2(x[0], x[1]);
          }
          op[tt] = __builtin_bit_cast(bf16x8, wv);
        }
      };
      auto step = [&](int qb, int qn) __attribute__((always_inline)) {
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) tb[tt][cb] = ld_t(qb, tt, cb);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          sc = bwd_mfma(qa[kk], lds16(&kv[0][c_off + kk * 2 * BR * 8]), sc);
          qa[kk] = ld_q(qn, kk);
          if (!DV) {
            dp = bwd_mfma(da[kk], lds16(&kv[DV ? 0 : 1][c_off + kk * 2 * BR * 8]), dp);
            da[kk] = ld_d(qn, kk);
          }
        }
        const int rel = BR * (qb - kb) + delta;
        const bool masked = !key_ok_all || (p.causal && rel < BR - 1);  // wave-uniform
        const int thr = !key_ok ? 32 : (p.causal && rel < BR - 1) ? l32 - 4 * hh - rel : 0;
        bf16x8 op[2];
        if (masked)
          probs(sc, dp, true, thr, op);
        else
          probs(sc, dp, false, thr, op);
        ld_rows(qn);
        // dv += P^T dO, dk += dS^T (q'/sqrt(D))
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            acc[cb] = bwd_mfma(op[tt], tb[tt][cb], acc[cb]);
          }
      };
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        qa[kk] = ld_q(p.NB - 1, kk);
        if (!DV) da[kk] = ld_d(p.NB - 1, kk);
      }
      ld_rows(p.NB - 1);
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
  // One query block per wave, the heaviest first (causal query block qb sees qb + 1 key blocks):
  // the grid's rounds run from qb = NB - 1 down and the last, partial round holds the lightest.
  const int qb_rank = blockIdx.x / (p.B * p.Hq);
  const int qunit = blockIdx.x % (p.B * p.Hq);  // b * Hq + h
  const int h = qunit % p.Hq, b = qunit / p.Hq;
  const int g = h / p.G;
  const size_t kunit = (size_t)b * p.Hkv + g;
  const int c_off = hh * BR * 8 + l32 * 8;
  const int delta = p.q_pos0 - p.k_pos0;

  {
    const int qb = p.NB - 1 - qb_rank;
    const size_t qtile = ((size_t)qunit * p.NB + qb) * T;
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
    // the moving key block's operands, one register set: each register is reloaded with the
    // next block's operand as soon as its MFMA has read it
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
        st = bwd_mfma(ka[kk], lds16(&qd[0][c_off + kk * 2 * BR * 8]), st);
        ka[kk] = ld_k(kn, kk);
        dpt = bwd_mfma(va[kk], lds16(&qd[1][c_off + kk * 2 * BR * 8]), dpt);
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
    if (kb_end > 0) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        ka[kk] = ld_k(0, kk);
        va[kk] = ld_v(0, kk);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) kt[tt][cb] = ld_t(0, tt, cb);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      for (int kb = 0; kb < kb_end; ++kb) {
        step(kb, min(kb + 1, kb_end - 1));
        __builtin_amdgcn_s_waitcnt(0x0F70);
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

hipError_t launch_bwd_d256_main(const BwdParams &p, const RopeTable &tab, hipStream_t stream) {
  const dim3 kv_grid((unsigned)((long long)p.B * p.Hkv * p.HS * p.NB));
  const dim3 q_grid((unsigned)((long long)p.B * p.Hq * p.NB));
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
