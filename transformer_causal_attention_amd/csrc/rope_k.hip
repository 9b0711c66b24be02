// Rotary embedding of the keys, once per key, into a head-major padded buffer.
//
// Rotation (half-split form): for pair i < D/2 at position p with angle a = p * theta_i,
//   k'_i = k_i cos a - k_{i+D/2} sin a,   k'_{i+D/2} = k_{i+D/2} cos a + k_i sin a
// i.e. x*cos + rotate_half(x)*sin with rotate_half = cat(-x2, x1) (Picotron page, section 1),
// theta_i = rope_theta^(-2i/D) (PaLM page, section 2.3).
//
// Every query block of the attention kernel re-reads the keys of all earlier blocks, so
// rotating them here once (instead of in every workgroup that stages them) keeps the
// attention loop free of trigonometry.  The output layout (B, Hkv, S_pad, D) makes each
// 64-key tile one contiguous run of memory; rows S .. S_pad-1 are written as zeros so the
// attention kernel never reads past the buffer.
//
// Thread layout: D/16 consecutive lanes share a key row, each rotating 8 pairs (16 bytes of
// each half), so a wave reads and writes whole rows.  The angle is formed in double
// precision and reduced to a fraction of a turn before the hardware sin/cos (which take
// turns and are accurate to ~1.2e-7 there).

#include "attn_device.h"

namespace attn {

template <int D>
__global__ void __launch_bounds__(256) rope_k_kernel(RopeKParams p, RopeTable tab) {
  constexpr int LPR = D / 16;  // lanes per key row
  __shared__ double freq[D / 2];
  if (threadIdx.x < D / 2) freq[threadIdx.x] = tab.rev[threadIdx.x];
  __syncthreads();

  const int rows_per_blk = 256 / LPR;
  const int n_rblk = (p.S_pad + rows_per_blk - 1) / rows_per_blk;
  const int unit = blockIdx.x / n_rblk;  // (b, g)
  const int j = (blockIdx.x % n_rblk) * rows_per_blk + threadIdx.x / LPR;
  const int c0 = 8 * (threadIdx.x % LPR);
  if (j >= p.S_pad) return;
  const int g = unit % p.Hkv;
  const int b = unit / p.Hkv;

  u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
  if (j < p.S) {
    const __bf16 *src = p.k + (((size_t)b * p.S + j) * p.Hkv + g) * D;
    lo = *reinterpret_cast<const u32x4 *>(src + c0);
    hi = *reinterpret_cast<const u32x4 *>(src + c0 + D / 2);
    u32x4 olo, ohi;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float t0 = turn_fraction(j, freq[c0 + 2 * w]);
      const float t1 = turn_fraction(j, freq[c0 + 2 * w + 1]);
      const float s0 = __builtin_amdgcn_sinf(t0), cs0 = __builtin_amdgcn_cosf(t0);
      const float s1 = __builtin_amdgcn_sinf(t1), cs1 = __builtin_amdgcn_cosf(t1);
      const float x0 = bf16_lo(lo[w]), x1 = bf16_hi(lo[w]);
      const float y0 = bf16_lo(hi[w]), y1 = bf16_hi(hi[w]);
      olo[w] = pack_bf16x2(x0 * cs0 - y0 * s0, x1 * cs1 - y1 * s1);
      ohi[w] = pack_bf16x2(y0 * cs0 + x0 * s0, y1 * cs1 + x1 * s1);
    }
    lo = olo;
    hi = ohi;
  }
  __bf16 *dst = p.kr + (((size_t)b * p.Hkv + g) * p.S_pad + j) * D;
  *reinterpret_cast<u32x4 *>(dst + c0) = lo;
  *reinterpret_cast<u32x4 *>(dst + c0 + D / 2) = hi;
}

template <int D>
hipError_t launch_rope_k(const RopeKParams &p, const RopeTable &tab, hipStream_t stream) {
  const int rows_per_blk = 256 / (D / 16);
  const int n_rblk = (p.S_pad + rows_per_blk - 1) / rows_per_blk;
  const long long blocks = (long long)p.B * p.Hkv * n_rblk;
  hipLaunchKernelGGL(rope_k_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, stream, p, tab);
  return hipGetLastError();
}

template hipError_t launch_rope_k<64>(const RopeKParams &, const RopeTable &, hipStream_t);
template hipError_t launch_rope_k<128>(const RopeKParams &, const RopeTable &, hipStream_t);

}  // namespace attn
