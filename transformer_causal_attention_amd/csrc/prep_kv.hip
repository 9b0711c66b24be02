// Key/value preparation, once per key: rotary embedding of K and transposition of V, into
// head-major buffers padded to whole 64-key tiles.
//
// Rotation (half-split form): for pair i < D/2 at position p = k_pos0 + j (the shard's first
// key position plus the row) with angle a = p * theta_i,
//   k'_i = k_i cos a - k_{i+D/2} sin a,   k'_{i+D/2} = k_{i+D/2} cos a + k_i sin a
// i.e. x*cos + rotate_half(x)*sin with rotate_half = cat(-x2, x1) (Picotron page, section 1),
// theta_i = rope_theta^(-2i/D) (PaLM page, section 2.3).  Values are not rotated.  In the
// adjacent-pair form the keys are read with their dims reordered (evens, then odds) and then
// rotated as above.
//
// Every query block of the attention kernel re-reads the keys and values of all earlier
// blocks, so doing this work here once keeps the attention loop free of trigonometry and of
// transposing loads.  Both outputs are stored as whole 64-key tiles of TB = 64*D*2 bytes in
// "chunk-major" order, so that the attention kernel copies a tile to LDS as one contiguous run
// and every MFMA operand it needs is one 16-byte LDS read at (per-lane base + constant):
//   kr tile: [D/8 dimension chunks][64 keys][8 dims]  (rotated keys)
//   vt tile: [8 key chunks][D columns][8 keys]        (values, transposed)
// Inside every group of 16 keys the key positions of vt are permuted by swapping bits 2 and 3
// of the key index, which is the key order in which the score accumulators hand the
// probabilities to the P.V product (see the attention kernel).  Tiles cover (B, Hkv, S_pad/64)
// and keys S .. S_pad-1 are written as zeros, so the attention kernel reads whole tiles.
// The angle is formed in double precision and reduced to a fraction of a turn before the
// hardware sin/cos (which take turns and are accurate to ~1.2e-7 there).

#include "attn_device.h"

namespace attn {

template <int D>
__global__ void __launch_bounds__(256) prep_kv_kernel(PrepParams p, RopeTable tab) {
  constexpr int VSTR = D + 8;  // staged value row, elements (16-byte aligned rows)
  __shared__ double freq[D / 2];
  __shared__ __attribute__((aligned(16))) uint16_t vs[64 * VSTR];
  const int tid = threadIdx.x;

  const int n_tiles = p.S_pad / 64;       // tiles per (b, g) in the output layout
  const int unit = blockIdx.x / p.n_run;  // (b, g)
  const int j0 = (p.tile0 + blockIdx.x % p.n_run) * 64;
  const int g = unit % p.Hkv;
  const int b = unit / p.Hkv;
  const size_t src_rs = (size_t)p.Hkv * D;  // elements between consecutive keys in k, v
  const __bf16 *ksrc = p.k + ((size_t)b * p.S_rows * p.Hkv + g) * D;
  const __bf16 *vsrc = p.v + ((size_t)b * p.S_rows * p.Hkv + g) * D;

  // Every load of the tile is issued before any of them is used, so the block waits for memory
  // once.  Rows past S load row S-1 (in bounds) and are replaced by zeros afterwards.
  // Keys: 64 keys x D/16 pairs of 8-dimension chunks (c, c + D/2); lanes walk keys, so each
  // chunk row of the tile is written contiguously.
  constexpr int NKI = D / 64;  // key items per thread
  constexpr int NVI = D / 32;  // value items per thread: 64 rows x D/8 chunks
  u32x4 kl[NKI], kh[NKI], vv[NVI];
#pragma unroll
  for (int it = 0; it < NKI; ++it) {
    const int item = tid + 256 * it;
    const int j = min(j0 + item % 64, p.S - 1);
    if (tab.interleaved) {  // dims 16c .. 16c+15, split into evens and odds below
      const __bf16 *src = ksrc + (size_t)j * src_rs + 16 * (item / 64);
      kl[it] = *reinterpret_cast<const u32x4 *>(src);
      kh[it] = *reinterpret_cast<const u32x4 *>(src + 8);
    } else {
      const __bf16 *src = ksrc + (size_t)j * src_rs + 8 * (item / 64);
      kl[it] = *reinterpret_cast<const u32x4 *>(src);
      kh[it] = *reinterpret_cast<const u32x4 *>(src + D / 2);
    }
  }
#pragma unroll
  for (int it = 0; it < NVI; ++it) {
    const int item = tid + 256 * it;
    const int j = min(j0 + item / (D / 8), p.S - 1);
    vv[it] = *reinterpret_cast<const u32x4 *>(vsrc + (size_t)j * src_rs + 8 * (item % (D / 8)));
  }
  if (tid < D / 2) freq[tid] = tab.rev[tid];
  // values -> LDS (zeros past S)
#pragma unroll
  for (int it = 0; it < NVI; ++it) {
    const int item = tid + 256 * it;
    const int row = item / (D / 8);
    const u32x4 w = j0 + row < p.S ? vv[it] : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4 *>(vs + row * VSTR + 8 * (item % (D / 8))) = w;
  }
  __syncthreads();  // frequencies and staged values visible to every thread

  const size_t tile = ((size_t)b * p.Hkv + g) * n_tiles + (size_t)(j0 / 64);
  char *kdst = reinterpret_cast<char *>(p.kr) + tile * (64 * D * 2);
  char *vdst = reinterpret_cast<char *>(p.vt) + tile * (64 * D * 2);

  // rotated keys
#pragma unroll
  for (int it = 0; it < NKI; ++it) {
    const int item = tid + 256 * it;
    const int row = item % 64;
    const int cp = item / 64;  // chunk of the first half: dims 8cp .. 8cp+7
    const int c0 = 8 * cp;
    const int j = j0 + row;
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    u32x4 xk = kl[it], yk = kh[it];  // dims 8cp + e and D/2 + 8cp + e (after the reordering)
    if (tab.interleaved) deinterleave16(kl[it], kh[it], xk, yk);
    if (j < p.S) {  // keys past S stay zero
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float t0 = turn_fraction(p.k_pos0 + j, freq[c0 + 2 * w]);
        const float t1 = turn_fraction(p.k_pos0 + j, freq[c0 + 2 * w + 1]);
        // (hardware sin/cos take turns)
        const u32x2 r = rotate_packed(xk[w], yk[w], __builtin_amdgcn_cosf(t0), __builtin_amdgcn_sinf(t0),
                                      __builtin_amdgcn_cosf(t1), __builtin_amdgcn_sinf(t1));
        lo[w] = r[0];
        hi[w] = r[1];
      }
    }
    *reinterpret_cast<u32x4 *>(kdst + (size_t)cp * 1024 + row * 16) = lo;
    *reinterpret_cast<u32x4 *>(kdst + (size_t)(cp + D / 16) * 1024 + row * 16) = hi;
  }

  // transposed values: key chunk q (positions 8q .. 8q+7, holding keys swap23(position)) of
  // column c; lanes walk columns
#pragma unroll
  for (int it = 0; it < D / 32; ++it) {
    const int item = tid + 256 * it;  // 8 key chunks x D columns
    const int c = item % D;
    const int q = item / D;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p0 = 8 * q + 2 * e;
      const int r0 = (p0 & ~12) | ((p0 & 4) << 1) | ((p0 & 8) >> 1);
      const int r1 = r0 + 1;  // bit 0 is not permuted
      w[e] = (uint32_t)vs[r0 * VSTR + c] | ((uint32_t)vs[r1 * VSTR + c] << 16);
    }
    *reinterpret_cast<u32x4 *>(vdst + (size_t)q * (D * 16) + c * 16) = w;
  }
}

template <int D>
hipError_t launch_prep_kv(const PrepParams &p, const RopeTable &tab, hipStream_t stream) {
  const long long blocks = (long long)p.B * p.Hkv * p.n_run;
  hipLaunchKernelGGL(prep_kv_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, stream, p, tab);
  return hipGetLastError();
}

template hipError_t launch_prep_kv<64>(const PrepParams &, const RopeTable &, hipStream_t);
template hipError_t launch_prep_kv<128>(const PrepParams &, const RopeTable &, hipStream_t);
template hipError_t launch_prep_kv<256>(const PrepParams &, const RopeTable &, hipStream_t);

}  // namespace attn
