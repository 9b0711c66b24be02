// Fused causal attention forward in float32 (inputs, arithmetic and outputs), for gfx950.
//
// Same definition as the bf16 kernel -- half-split rotary embedding of q and k (Picotron
// page, section 1; PaLM page, section 2.3), scores / sqrt(head_dim), later keys masked,
// softmax over keys with the running maximum subtracted, lse = ln sum exp(score)
// (llama3-from-scratch page; PaLM page, section 2.5) -- evaluated tile by tile with an
// online softmax so no score matrix is stored.  There is no float32 MFMA path here: this
// kernel serves precision (float32 end to end), so one lane owns one query row and does
// plain FMAs against key/value tiles staged in LDS, where every lane reads the same key
// at the same time (LDS broadcast).  Keys are rotated while they are staged.

#include <hip/hip_ext.h>

#include "attn_device.h"

namespace attn {

constexpr int F32_TK = 32;  // keys per staged tile
constexpr int F32_SUB = 8;  // keys per softmax update

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64) attn_fwd_f32_kernel(F32Params p, RopeTable tab) {
  // rows padded by 4 floats: 16-byte aligned for 4-wide broadcast reads, and the staging
  // writes (one key row per lane) spread over the banks
  __shared__ __attribute__((aligned(16))) float ks[F32_TK][D + 4];
  __shared__ __attribute__((aligned(16))) float vs[F32_TK][D + 4];

  const int lane = threadIdx.x;
  const int rb = blockIdx.x % p.n_row_blocks;
  const int bh = blockIdx.x / p.n_row_blocks;
  const int head = bh % p.Hq;
  const int b = bh / p.Hq;
  const int g = head / p.G;
  const int S = p.S;
  const int row = rb * 64 + lane;
  const int delta = p.q_pos0 - p.k_pos0;  // key j is visible to query i iff j <= i + delta
  const int kv_end = CAUSAL ? max(0, min(S, min(S, rb * 64 + 64) + delta)) : S;

  // rotated, pre-scaled query row in registers
  float q[D];
  {
    const float *src = p.q + (((size_t)b * S + min(row, S - 1)) * p.Hq + head) * D;
#pragma unroll
    for (int c = 0; c < D / 2; ++c) {
      float sn, cs;
      sincos_turns(turn_fraction(p.q_pos0 + row, tab.rev[c]), &sn, &cs);
      // pair (c, c + D/2), or (2c, 2c + 1) in the adjacent-pair form
      const float x = row < S ? src[rope_src_dim(c, D / 2, tab.interleaved)] : 0.f;
      const float y = row < S ? src[rope_src_dim(c + D / 2, D / 2, tab.interleaved)] : 0.f;
      q[c] = (x * cs - y * sn) * p.q_scale;
      q[c + D / 2] = (y * cs + x * sn) * p.q_scale;
    }
  }

  float o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int kbase = 0; kbase < kv_end; kbase += F32_TK) {
    __syncthreads();  // previous tile fully consumed
    {
      const int t = lane & (F32_TK - 1);
      const int j = kbase + t;
      if (lane < F32_TK) {  // lanes 0..31 stage rotated keys
        const float *src = p.k + (((size_t)b * S + min(j, S - 1)) * p.Hkv + g) * D;
#pragma unroll 4
        for (int c = 0; c < D / 2; ++c) {
          float sn, cs;
          sincos_turns(turn_fraction(p.k_pos0 + j, tab.rev[c]), &sn, &cs);
          const float x = j < S ? src[rope_src_dim(c, D / 2, tab.interleaved)] : 0.f;
          const float y = j < S ? src[rope_src_dim(c + D / 2, D / 2, tab.interleaved)] : 0.f;
          ks[t][c] = x * cs - y * sn;
          ks[t][c + D / 2] = y * cs + x * sn;
        }
      } else {  // lanes 32..63 stage values
        const float *src = p.v + (((size_t)b * S + min(j, S - 1)) * p.Hkv + g) * D;
#pragma unroll 8
        for (int c = 0; c < D; ++c) vs[t][c] = j < S ? src[c] : 0.f;
      }
    }
    __syncthreads();

    const int tile_end = min(F32_TK, kv_end - kbase);
    for (int j0 = 0; j0 < tile_end; j0 += F32_SUB) {
      float s[F32_SUB];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < F32_SUB; ++u) {
        const int jl = j0 + u;
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < D; c += 4) {
          const f32x4 k4 = *reinterpret_cast<const f32x4 *>(&ks[jl][c]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = fmaf(q[c + e], k4[e], acc);
        }
        const int j = kbase + jl;
        const bool masked = jl >= tile_end || j >= S || (CAUSAL && j > row + delta);
        s[u] = masked ? -INFINITY : acc;
        mx = fmaxf(mx, s[u]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float rsum = 0.f;
#pragma unroll
      for (int u = 0; u < F32_SUB; ++u) {
        s[u] = exp2f(s[u] - m_use);
        rsum += s[u];
      }
      l_run = l_run * alpha + rsum;
      m_run = m_new;
#pragma unroll
      for (int c = 0; c < D; c += 4) {
        f32x4 acc = {o[c] * alpha, o[c + 1] * alpha, o[c + 2] * alpha, o[c + 3] * alpha};
#pragma unroll
        for (int u = 0; u < F32_SUB; ++u) {
          const f32x4 v4 = *reinterpret_cast<const f32x4 *>(&vs[j0 + u][c]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = fmaf(s[u], v4[e], acc[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) o[c + e] = acc[e];
      }
    }
  }

  if (row < S) {
    // a row with no visible key (a shard of later keys) has out 0 and lse -inf
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float *dst = p.out + (((size_t)b * S + row) * p.Hq + head) * D;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      f32x4 w4 = {o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
      *reinterpret_cast<f32x4 *>(dst + c) = w4;
    }
    p.lse[((size_t)b * p.Hq + head) * S + row] = l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_attn_f32(const F32Params &p, const RopeTable &tab, hipStream_t stream,
                            hipEvent_t ev_start, hipEvent_t ev_stop) {
  const long long blocks = (long long)p.B * p.Hq * p.n_row_blocks;
  hipExtLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(64), 0, stream,
                        ev_start, ev_stop, 0, p, tab);
  return hipGetLastError();
}

template hipError_t launch_attn_f32<64, true>(const F32Params &, const RopeTable &, hipStream_t,
                                                    hipEvent_t, hipEvent_t);
template hipError_t launch_attn_f32<64, false>(const F32Params &, const RopeTable &, hipStream_t,
                                                    hipEvent_t, hipEvent_t);
template hipError_t launch_attn_f32<128, true>(const F32Params &, const RopeTable &, hipStream_t,
                                                    hipEvent_t, hipEvent_t);
template hipError_t launch_attn_f32<128, false>(const F32Params &, const RopeTable &, hipStream_t,
                                                    hipEvent_t, hipEvent_t);

}  // namespace attn
