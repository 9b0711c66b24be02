// Decode step: one new query row per (batch row, query head) attending to a key/value cache,
// for gfx950.  Same definition as the forward (RoPE on q and k, scores / sqrt(head_dim), keys
// after the query masked, stable softmax, lse; Picotron, PaLM and llama3-from-scratch pages),
// restricted to the single row at position q_pos -- the generation loop of the PaLM page
// (section 2.5 notes that a shared K/V head makes this step cheaper) appends one token at a
// time and attends it to every cached key.
//
// The cache is kept in the preparation pass's tile layout (rotated keys, transposed values,
// 64-key tiles), so every MFMA operand is one 16-byte LDS read as in the forward kernel, and
// a new token only re-prepares the last tile.  The step is HBM-bound: every cached key and
// value is read once.  The key range is split over workgroups (split-K), each leaves a
// partial (o, m, l) for its keys, and a second kernel joins the partials by their maxima.
//
// A workgroup is one wave: it holds the 32 query heads of a head block (the G heads sharing
// the K/V head, 32 at a time) as the columns of the MFMA operand Q^T, so S^T = K Q^T puts one
// head per lane and each staged tile serves every head of the group.  Tiles are copied to
// LDS with buffer_load ... lds, two in flight.

#include "attn_device.h"

#define LDS_AS __attribute__((address_space(3)))

namespace attn {

namespace {

constexpr int DBN = 64;  // keys per tile

__device__ __forceinline__ float dec_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

__device__ __forceinline__ float dec_max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ f32x16 dec_mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

template <int D>
__global__ void __launch_bounds__(64) attn_decode_kernel(DecodeParams p, RopeTable tab) {
  constexpr int NKK = D / 16;
  constexpr int NCB = D / 32;
  constexpr int TB = DBN * D * 2;  // bytes of one K or V^T tile
  // [buffer][K tile, V^T tile]
  __shared__ __attribute__((aligned(1024))) char lds[2][2][TB];

  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // workgroup -> (b, g, head block, split)
  int w = blockIdx.x;
  const int split = w % p.n_split;
  w /= p.n_split;
  const int hb = w % p.n_hblk;
  w /= p.n_hblk;
  const int g = w % p.Hkv;
  const int b = w / p.Hkv;

  const int n_keys = p.q_pos + 1;  // keys 0 .. q_pos are visible
  const int t_begin = split * p.tiles_per_split;
  const int t_end = min((n_keys + DBN - 1) / DBN, t_begin + p.tiles_per_split);

  const size_t n_tiles = (size_t)(p.S_pad / DBN);
  const size_t unit_bytes = n_tiles * TB;
  const char *kr_tiles = reinterpret_cast<const char *>(p.kr) + ((size_t)b * p.Hkv + g) * unit_bytes;
  const char *vt_tiles = reinterpret_cast<const char *>(p.vt) + ((size_t)b * p.Hkv + g) * unit_bytes;
  const __amdgpu_buffer_rsrc_t kr_buf =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kr_tiles), 0, (int)unit_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vt_buf =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(vt_tiles), 0, (int)unit_bytes, 0x00020000);
  const uint32_t dma_lane = 16u * (uint32_t)lane;
  auto stage = [&](int t, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < TB / 1024; ++r) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr_buf, (LDS_AS void *)(lds[buf][0] + r * 1024), 16, dma_lane,
                                               (uint32_t)t * TB + r * 1024, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vt_buf, (LDS_AS void *)(lds[buf][1] + r * 1024), 16, dma_lane,
                                               (uint32_t)t * TB + r * 1024, 0, 0);
    }
  };
  if (t_begin < t_end) stage(t_begin, 0);

  // Q^T operand: lane l holds head column l % 32 (zeros past the group), dimensions 16kk + 8hh
  // + e, rotated at q_pos and scaled by log2(e)/sqrt(D)
  const int hc = hb * 32 + l32;  // head within the group
  const bool head_ok = hc < p.G;
  const int head = g * p.G + hc;
  bf16x8 qf[NKK];
  {
    u32x4 raw[NKK];
    const __bf16 *src = p.q + ((size_t)b * p.Hq + (head_ok ? head : 0)) * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      raw[kk] = head_ok ? *reinterpret_cast<const u32x4 *>(src + 16 * kk) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int kk = 0; kk < NKK / 2; ++kk) {
      u32x4 olo, ohi;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) {
        float r[2][2];
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const int e = 2 * wv + z;
          const float t = turn_fraction(p.q_pos, tab.rev[16 * kk + 8 * hh + e]);
          const float sn = __builtin_amdgcn_sinf(t), cs = __builtin_amdgcn_cosf(t);  // turns
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
  }

  f32x16 o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{};
  float m_run = -INFINITY;  // running maximum of the base-2 scores of this lane's head
  float l_run = 0.f;        // this lane half's share of the running sum

  const int k_lane = hh * 1024 + l32 * 16;
  const int v_lane = hh * 16 * D + l32 * 16;
  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile t is in LDS; the other buffer's reads of the previous step are done
    if (t + 1 < t_end) stage(t + 1, buf ^ 1);
    const char *kd = lds[buf][0];
    const char *vd = lds[buf][1];
    const int kb0 = t * DBN;
    f32x16 sc[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      sc[jb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        sc[jb] = dec_mfma(*reinterpret_cast<const bf16x8 *>(kd + k_lane + 2 * kk * 1024 + jb * 512), qf[kk], sc[jb]);
    }
    if (kb0 + DBN - 1 > p.q_pos) {  // keys after the query
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (kb0 + 32 * jb + 8 * (v >> 2) + 4 * hh + (v & 3) > p.q_pos) sc[jb][v] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[jb][v]);
    mx = dec_max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);  // finite: key kb0 <= q_pos is in every tile
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float rs = 0.f;
    bf16x8 pk[2][2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        u32x4 wd;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const float e0 = __builtin_amdgcn_exp2f(sc[jb][8 * tt + 2 * ww] - m_new);
          const float e1 = __builtin_amdgcn_exp2f(sc[jb][8 * tt + 2 * ww + 1] - m_new);
          rs += e0 + e1;
          wd[ww] = pack_bf16x2(e0, e1);
        }
        pk[jb][tt] = __builtin_bit_cast(bf16x8, wd);
      }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          o[cb] = dec_mfma(*reinterpret_cast<const bf16x8 *>(vd + v_lane + (4 * jb + 2 * tt) * 16 * D + cb * 512),
                           pk[jb][tt], o[cb]);
  }

  // partial result of this split: o as [split-row][32 heads][D] floats, m and l per head
  const size_t prow = (((size_t)b * p.Hkv + g) * p.n_hblk + hb) * p.n_split + split;
  float *po = p.po + (prow * 32 + l32) * D;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4)
      *reinterpret_cast<f32x4 *>(po + 32 * cb + 8 * v4 + 4 * hh) =
          f32x4{o[cb][4 * v4], o[cb][4 * v4 + 1], o[cb][4 * v4 + 2], o[cb][4 * v4 + 3]};
  const float l_tot = l_run + dec_xor32(l_run);
  if (hh == 0) {
    p.pm[prow * 32 + l32] = m_run;
    p.pl[prow * 32 + l32] = l_tot;
  }
}

// Joins the splits of every (b, head): m = max m_i, l = sum l_i 2^(m_i - m),
// out = sum o_i 2^(m_i - m) / l (bf16), lse = ln 2 * (m + log2 l).  32 threads per head, each
// owning D/32 consecutive dimensions.
template <int D>
__global__ void __launch_bounds__(256) attn_decode_join_kernel(DecodeParams p) {
  constexpr int E = D / 32;
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long bh = t / 32;  // (b, head)
  if (bh >= (long long)p.B * p.Hq) return;
  const int part = (int)(t % 32);
  const int head = (int)(bh % p.Hq);
  const int b = (int)(bh / p.Hq);
  const int g = head / p.G;
  const int hc = head % p.G;
  const int hb = hc / 32;
  const size_t row0 = (((size_t)b * p.Hkv + g) * p.n_hblk + hb) * p.n_split;
  const int n_used = min(p.n_split, ((p.q_pos + 1 + DBN - 1) / DBN + p.tiles_per_split - 1) / p.tiles_per_split);
  float m = -INFINITY;
  for (int s = 0; s < n_used; ++s) m = fmaxf(m, p.pm[(row0 + s) * 32 + hc % 32]);
  float l = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int s = 0; s < n_used; ++s) {
    const size_t r = (row0 + s) * 32 + hc % 32;
    const float c = __builtin_amdgcn_exp2f(p.pm[r] - m);
    l += p.pl[r] * c;
    const float *src = p.po + r * D + part * E;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += src[e] * c;
  }
  const float inv = 1.0f / l;
  __bf16 *dst = p.out + ((size_t)b * p.Hq + head) * D + part * E;
#pragma unroll
  for (int e = 0; e < E; e += 2) *reinterpret_cast<uint32_t *>(dst + e) = pack_bf16x2(acc[e] * inv, acc[e + 1] * inv);
  if (part == 0) p.lse[(size_t)b * p.Hq + head] = (m + __log2f(l)) * 0.69314718055994531f;
}

template <int D>
hipError_t launch_decode(const DecodeParams &p, const RopeTable &tab, hipStream_t stream) {
  const long long wgs = (long long)p.B * p.Hkv * p.n_hblk * p.n_split;
  hipLaunchKernelGGL(attn_decode_kernel<D>, dim3((unsigned)wgs), dim3(64), 0, stream, p, tab);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long long threads = (long long)p.B * p.Hq * 32;
  hipLaunchKernelGGL(attn_decode_join_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template hipError_t launch_decode<64>(const DecodeParams &, const RopeTable &, hipStream_t);
template hipError_t launch_decode<128>(const DecodeParams &, const RopeTable &, hipStream_t);

}  // namespace attn
