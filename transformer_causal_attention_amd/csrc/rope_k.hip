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

#include "attn_device.h"

namespace attn {

// One thread per key row and 8-pair chunk.  The chunk index comes from blockIdx, so it is
// uniform across the workgroup and the frequency table is read with scalar loads.
template <int D>
__global__ void __launch_bounds__(256) rope_k_kernel(RopeKParams p, RopeTable tab) {
  constexpr int NC = D / 16;  // chunks of 8 rotation pairs
  const int chunk = blockIdx.x % NC;
  const int rblk = blockIdx.x / NC;
  const int n_rblk = (p.S_pad + 255) / 256;
  const int unit = rblk / n_rblk;  // (b, g)
  const int j = (rblk % n_rblk) * 256 + threadIdx.x;
  if (j >= p.S_pad) return;
  const int g = unit % p.Hkv;
  const int b = unit / p.Hkv;
  const int c0 = chunk * 8;

  u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
  if (j < p.S) {
    const __bf16 *src = p.k + (((size_t)b * p.S + j) * p.Hkv + g) * D;
    lo = *reinterpret_cast<const u32x4 *>(src + c0);
    hi = *reinterpret_cast<const u32x4 *>(src + c0 + D / 2);
    u32x4 olo, ohi;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float x0 = bf16_lo(lo[w]), x1 = bf16_hi(lo[w]);
      float y0 = bf16_lo(hi[w]), y1 = bf16_hi(hi[w]);
      float s0, cs0, s1, cs1;
      sincos_turns(turn_fraction(j, tab.rev[c0 + 2 * w]), &s0, &cs0);
      sincos_turns(turn_fraction(j, tab.rev[c0 + 2 * w + 1]), &s1, &cs1);
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
  const int n_rblk = (p.S_pad + 255) / 256;
  const long long blocks = (long long)p.B * p.Hkv * n_rblk * (D / 16);
  hipLaunchKernelGGL(rope_k_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, stream, p, tab);
  return hipGetLastError();
}

template hipError_t launch_rope_k<64>(const RopeKParams &, const RopeTable &, hipStream_t);
template hipError_t launch_rope_k<128>(const RopeKParams &, const RopeTable &, hipStream_t);

}  // namespace attn
