// Fused causal attention forward for head_dim 256, bf16 in / bf16 out, fp32 accumulation, gfx950.
//
// Same definition as the head_dim 64 / 128 kernel (rotary embedding of q and k, scores divided
// by sqrt(head_dim), later keys masked, softmax with the row maximum subtracted, lse; Picotron,
// llama3-from-scratch and PaLM pages), for the head size of the PaLM page's largest model
// (section 4: 256 per head, multi-query).  At d = 256 the other kernel's staging (two wave groups,
// each with double-buffered 64-key K and V^T tiles in LDS, and 32 rows x d of accumulators per
// wave at two waves per SIMD) would need 256 KiB of LDS and more registers than two waves per
// SIMD have, so this kernel is built the simple way:
//
//   - one wave per workgroup owns 32 query rows of one head (heavy row blocks are dispatched
//     first, so the causal staircase fills the GPU evenly);
//   - the queries are loaded, rotated in registers and scaled by log2(e)/16 once;
//   - the prepared keys and values (the preparation pass's 64-key tiles: rotated K chunk-major,
//     V transposed) stream from L2/HBM straight into registers, 32 keys at a time, with the next
//     32 keys' loads issued while the current ones are used;
//   - S^T = K Q^T and O^T = V^T P^T on the 32x32x16 bf16 MFMA (the accumulator layouts of the
//     decode kernel), an exact running maximum per 32 keys, and the rescale of o and l.
//
// Keys above the diagonal are never loaded.  Rows with no visible key (only in a shard of later
// keys) give out 0 and lse -inf.

#include <hip/hip_ext.h>

#include "attn_device.h"

namespace attn {

namespace {

__device__ __forceinline__ float d256_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

__device__ __forceinline__ float d256_max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ f32x16 d256_mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

template <bool CAUSAL>
__global__ void __launch_bounds__(64) attn_fwd_d256_kernel(FwdParams p, RopeTable tab) {
  constexpr int D = 256;
  constexpr int NKK = D / 16;     // MFMA steps over head_dim
  constexpr int NCB = D / 32;     // 32-column blocks of the output
  constexpr int TB = 64 * D * 2;  // bytes of one prepared 64-key tile

  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // workgroup -> (b, head, row block), heaviest row blocks first
  const int nrb = p.n_row_blocks;
  int w = blockIdx.x;
  const int rb = nrb - 1 - w % nrb;
  w /= nrb;
  const int head = w % p.Hq;
  const int b = w / p.Hq;
  const int g = head / p.G;
  const int S = p.S;
  const int delta = p.delta;
  const int row0 = rb * 32;
  const int my_row = row0 + l32;
  // keys the block sees: query i sees key j iff j <= i + delta (causal), j < S
  const int kend = CAUSAL ? max(0, min(S, min(S, row0 + 32) + delta)) : S;
  const int n_halves = (kend + 31) / 32;

  // ---- queries: lane holds dims 16kk + 8hh + e of row my_row in raw[kk] (evens / odds of a
  // 16-dim run in the adjacent-pair rotary form), rotated and scaled into the B operand Q^T
  u32x4 raw[NKK];
  if (my_row < S) {
    const __bf16 *row = p.q + (((size_t)b * S + my_row) * p.Hq + head) * D;
    if (tab.interleaved) {
#pragma unroll
      for (int kk = 0; kk < NKK / 2; ++kk) {
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(row + 32 * kk + 16 * hh);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(row + 32 * kk + 16 * hh + 8);
        deinterleave16(lo, hi, raw[kk], raw[kk + NKK / 2]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) raw[kk] = *reinterpret_cast<const u32x4 *>(row + 16 * kk + 8 * hh);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) raw[kk] = u32x4{0u, 0u, 0u, 0u};
  }

  // the (b, g) run of prepared tiles as buffer resources (S_pad * D * 2 < 2^31 bytes)
  const uint32_t unit_bytes = (uint32_t)(p.S_pad / 64) * TB;
  const size_t unit = (size_t)b * p.Hkv + g;
  const __amdgpu_buffer_rsrc_t kbuf = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(reinterpret_cast<const char *>(p.kr) + unit * unit_bytes), 0, (int)unit_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vbuf = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(reinterpret_cast<const char *>(p.vt) + unit * unit_bytes), 0, (int)unit_bytes, 0x00020000);
  // 32-key half h = keys 32h .. 32h+31: tile h/2, half h%2 of it.
  //   K (A operand of S^T = K Q^T): key 32(h%2) + l32, dims 16kk + 8hh .. +7 = chunk 2kk + hh
  //     at [chunk][64 keys][8] -> (2kk + hh) * 1024 + (32(h%2) + l32) * 16
  //   V^T (A operand of O^T = V^T P^T): column 32cb + l32, key chunk 4(h%2) + 2tt + hh
  //     at [8 key chunks][D columns][8] -> (4(h%2) + 2tt + hh) * 16D + (32cb + l32) * 16
  const uint32_t k_lane = (uint32_t)(hh * 1024 + l32 * 16);
  const uint32_t v_lane = (uint32_t)(hh * 16 * D + l32 * 16);
  bf16x8 kq[NKK], vq[2][NCB];
  auto load_k = [&](int h) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(h >> 1) * TB + (uint32_t)(h & 1) * 512 + k_lane;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      kq[kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kbuf, base + kk * 2048, 0, 0));
  };
  auto load_v = [&](int h) __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)(h >> 1) * TB + (uint32_t)(h & 1) * 4 * 16 * D + v_lane;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        vq[tt][cb] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vbuf, base + tt * 2 * 16 * D + cb * 512, 0, 0));
  };
  if (n_halves > 0) {
    load_k(0);
    load_v(0);
  }

  // rotation of pairs (c, c + D/2) at position q_pos0 + my_row, scaled by log2(e)/sqrt(D)
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK / 2; ++kk) {
    u32x4 olo, ohi;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) {
      float r[2][2];
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const int e = 2 * wv + z;
        const float t = turn_fraction(p.q_pos0 + my_row, tab.rev[16 * kk + 8 * hh + e]);
        const float sn = __builtin_amdgcn_sinf(t), cs = __builtin_amdgcn_cosf(t);  // argument in turns
        const uint32_t lo = raw[kk][wv], hi = raw[kk + NKK / 2][wv];
        const float xv = z ? bf16_hi(lo) : bf16_lo(lo);
        const float yv = z ? bf16_hi(hi) : bf16_lo(hi);
        r[0][z] = (xv * cs - yv * sn) * p.q_scale;
        r[1][z] = (yv * cs + xv * sn) * p.q_scale;
      }
      olo[wv] = pack_bf16x2(r[0][0], r[0][1]);
      ohi[wv] = pack_bf16x2(r[1][0], r[1][1]);
    }
    qf[kk] = __builtin_bit_cast(bf16x8, olo);
    qf[kk + NKK / 2] = __builtin_bit_cast(bf16x8, ohi);
  }

  f32x16 o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{};
  float m_run = -INFINITY;  // running maximum of this row's base-2 scores
  float l_run = 0.f;        // this lane half's share of the running sum

  for (int h = 0; h < n_halves; ++h) {
    f32x16 sc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) sc = d256_mfma(kq[kk], qf[kk], sc);
    if (h + 1 < n_halves) load_k(h + 1);
    // keys of this half held by the lane: 32h + 8(v>>2) + 4hh + (v&3)
    const int kb0 = 32 * h;
    if ((CAUSAL && kb0 + 31 > row0 + delta) || kb0 + 32 > S) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = kb0 + 8 * (v >> 2) + 4 * hh + (v & 3);
        if ((CAUSAL && j > my_row + delta) || j >= S) sc[v] = -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sc[v]);
    mx = d256_max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // a row with no visible key yet
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float rs = 0.f;
    bf16x8 pk[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      u32x4 wd;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float e0 = __builtin_amdgcn_exp2f(sc[8 * tt + 2 * ww] - m_use);
        const float e1 = __builtin_amdgcn_exp2f(sc[8 * tt + 2 * ww + 1] - m_use);
        rs += e0 + e1;
        wd[ww] = pack_bf16x2(e0, e1);
      }
      pk[tt] = __builtin_bit_cast(bf16x8, wd);
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) o[cb] = d256_mfma(vq[tt][cb], pk[tt], o[cb]);
    if (h + 1 < n_halves) load_v(h + 1);
  }

  // ---- out = o / l (lane: row my_row, dims 32cb + 8a + 4hh + 0..3), lse = ln 2 (m + log2 l)
  const float l_tot = l_run + d256_xor32(l_run);
  if (my_row < S) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
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
      p.lse[((size_t)b * p.Hq + head) * S + my_row] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

template <bool CAUSAL>
hipError_t launch_attn_d256(const FwdParams &p, const RopeTable &tab, hipStream_t stream, hipEvent_t ev_start,
                            hipEvent_t ev_stop) {
  const long long blocks = (long long)p.B * p.Hq * p.n_row_blocks;
  hipExtLaunchKernelGGL((attn_fwd_d256_kernel<CAUSAL>), dim3((unsigned)blocks), dim3(64), 0, stream, ev_start,
                        ev_stop, 0, p, tab);
  return hipGetLastError();
}

template hipError_t launch_attn_d256<true>(const FwdParams &, const RopeTable &, hipStream_t, hipEvent_t, hipEvent_t);
template hipError_t launch_attn_d256<false>(const FwdParams &, const RopeTable &, hipStream_t, hipEvent_t, hipEvent_t);

}  // namespace attn
