// Merge of two partial attention results over disjoint key sets, for gfx950.
//
// For each (batch row b, position s, head h): lse = ln(e^lse1 + e^lse2) and
// out = e^(lse1 - lse) * o1 + e^(lse2 - lse) * o2, the combination ring attention applies when
// each rank has attended its queries to one block of keys (Picotron page, "context
// parallelism and ring attention"); lse is the natural-log softmax denominator of each part.
// A part with lse = -inf (no visible key) contributes nothing; a row empty in both stays
// empty (out 0, lse -inf).
//
// Plain streaming work (HBM-bound): each thread owns 16 bytes of one row of o, the lanes of a
// row sit in one wave, so every lane reads the row's two lse values before any lane writes
// the merged one (out and lse may alias o1 and lse1, or o2 and lse2).

#include "attn_device.h"

namespace attn {

template <typename T>
__device__ __forceinline__ void load16(const void *p, float (&x)[16 / sizeof(T)]);

template <>
__device__ __forceinline__ void load16<__bf16>(const void *p, float (&x)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}

template <>
__device__ __forceinline__ void load16<float>(const void *p, float (&x)[4]) {
  const f32x4 w = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = w[i];
}

template <typename T>
__device__ __forceinline__ void store16(void *p, const float (&x)[16 / sizeof(T)]);

template <>
__device__ __forceinline__ void store16<__bf16>(void *p, const float (&x)[8]) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
  *reinterpret_cast<u32x4 *>(p) = w;
}

template <>
__device__ __forceinline__ void store16<float>(void *p, const float (&x)[4]) {
  *reinterpret_cast<f32x4 *>(p) = f32x4{x[0], x[1], x[2], x[3]};
}

template <typename T, int D>
__global__ void __launch_bounds__(256) attn_merge_kernel(MergeParams p) {
  constexpr int E = 16 / sizeof(T);  // elements per thread
  constexpr int TPR = D / E;         // threads per row (8 to 64: within one wave)
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = t / TPR;     // (b, s, h) in the (B, S, H) order of o
  if (row >= p.rows) return;
  const int part = (int)(t % TPR);
  const int h = (int)(row % p.H);
  const long long bs = row / p.H;
  const int s = (int)(bs % p.S);
  const long long b = bs / p.S;
  const long long li = (b * p.H + h) * p.S + s;  // lse is (B, H, S)

  const float l1 = p.lse1[li], l2 = p.lse2[li];
  const float mx = fmaxf(l1, l2);
  float lse = -INFINITY, w1 = 0.f, w2 = 0.f;
  if (mx != -INFINITY) {
    const float e1 = __expf(l1 - mx), e2 = __expf(l2 - mx);
    const float sum = e1 + e2;
    lse = mx + __logf(sum);
    w1 = e1 / sum;
    w2 = e2 / sum;
  }
  const size_t off = (size_t)row * D + (size_t)part * E;
  float x1[E], x2[E], y[E];
  load16<T>(static_cast<const T *>(p.o1) + off, x1);
  load16<T>(static_cast<const T *>(p.o2) + off, x2);
#pragma unroll
  for (int i = 0; i < E; ++i) y[i] = w1 * x1[i] + w2 * x2[i];
  store16<T>(static_cast<T *>(p.out) + off, y);
  if (part == 0) p.lse[li] = lse;
}

template <typename T, int D>
hipError_t launch_merge(const MergeParams &p, hipStream_t stream) {
  constexpr int TPR = D / (16 / sizeof(T));
  const long long threads = p.rows * TPR;
  const long long blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((attn_merge_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template hipError_t launch_merge<__bf16, 64>(const MergeParams &, hipStream_t);
template hipError_t launch_merge<__bf16, 128>(const MergeParams &, hipStream_t);
template hipError_t launch_merge<float, 64>(const MergeParams &, hipStream_t);
template hipError_t launch_merge<float, 128>(const MergeParams &, hipStream_t);
template hipError_t launch_merge<__bf16, 256>(const MergeParams &, hipStream_t);
template hipError_t launch_merge<float, 256>(const MergeParams &, hipStream_t);

}  // namespace attn
