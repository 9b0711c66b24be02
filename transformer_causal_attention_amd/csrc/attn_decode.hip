// Decode step: one new query row per (batch row, query head) attending to a key/value cache,
// for gfx950.  Same definition as the forward (RoPE on q and k, scores / sqrt(head_dim), keys
// after the query masked, stable softmax, lse; Picotron, PaLM and llama3-from-scratch pages),
// restricted to the single row at position q_pos -- the generation loop of the PaLM page
// (section 2.7) appends one token at a time and attends it to every cached key; section 2.5
// notes that a shared K/V head makes this step cheaper.
//
// The cache is kept in the preparation pass's tile layout (rotated keys, transposed values,
// 64-key tiles), so every MFMA operand is one 16-byte load at (per-lane base + constant), and a
// new token only re-prepares the last tile.  The step is HBM-bound: every cached key and value
// is read once and no tile is shared between waves, so tiles go straight from HBM into
// registers (no LDS), PD half tiles (32 keys) in flight per wave: the bytes in flight per CU are
// then bounded by the register file rather than by LDS.  The key range of each (b, K/V head) is
// split over waves (split-K); each leaves a partial (o, m, l) for its keys, and a second kernel
// joins the partials by their maxima.
//
// A workgroup holds the (up to) 32 query heads of a head block, the G heads that share the K/V
// head, 32 at a time, as the columns of the MFMA operand Q^T: S^T = K Q^T puts one head per lane
// and each loaded half tile serves every head of the block.  Up to head_dim 128 the workgroup is
// one wave.  At head_dim 256 the operands of one wave would not fit its registers, so the
// workgroup is two waves that split the dimensions: each takes half of the rotary pairs for the
// scores and half of the value columns for the output, the two partial score tiles are added
// through LDS, and both waves then run the same softmax on the same sums.

#include "attn_device.h"

namespace attn {

namespace {

constexpr int DBN = 64;  // keys per tile
#ifndef DECODE_DEPTH
#define DECODE_DEPTH 2
#endif
constexpr int kDecodeDepth = DECODE_DEPTH;  // half tiles in flight per wave
// A buffer offset past every cache run (runs are < 2^31 bytes); with the per-lane part added
// it stays below 2^31, so the range check sees it as out of bounds.
constexpr int kPastEnd = 0x7ff00000;

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

template <int D, int PD>
__global__ void __launch_bounds__(D == 256 ? 128 : 64) attn_decode_kernel(DecodeParams p, RopeTable tab) {
  constexpr int NW = D == 256 ? 2 : 1;  // waves per workgroup, splitting the dimensions
  constexpr int NKK = D / 16;           // k-steps of the full score product
  constexpr int NKW = NKK / NW;         // k-steps of this wave: NKW / 2 rotary pairs of chunks
  constexpr int NCB = D / 32 / NW;      // output column blocks of this wave
  constexpr int TB = DBN * D * 2;       // bytes of one K or V^T tile
  // partial score tiles of the two waves, double-buffered: [buffer][wave][quad][lane][4]
  __shared__ __attribute__((aligned(16))) float xs[NW > 1 ? 2 : 1][NW][4][64][4];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  // chunk pair j of this wave (j < NKW / 2) is the full product's pair wv * NKW / 2 + j; its two
  // chunks are k-steps kk_of(j) and kk_of(j) + NKK / 2 (the dimensions a rotation mixes)
  auto kk_of = [&](int j) __attribute__((always_inline)) {
    return (j / (NKW / 2)) * (NKK / 2) + wv * (NKW / 2) + j % (NKW / 2);
  };

  // workgroup -> (key range u = (b, g, split), head block).  With one head block, u is the
  // workgroup index.  With several, the head blocks of one key range read the same tiles: the
  // workgroups are dealt to the 8 XCDs round robin (workgroup i to XCD i % 8), so u's head
  // blocks are given indices 8 apart, i.e. neighbours on one XCD, and all but the first read
  // the tiles from that XCD's L2.  The grid is rounded up to whole groups of 8 key ranges and
  // the workgroups past the last range leave at once (before any barrier).
  int w, hb;
  if (p.n_hblk == 1) {
    w = blockIdx.x;
    hb = 0;
  } else {
    const int j = blockIdx.x / 8;
    hb = j % p.n_hblk;
    w = 8 * (j / p.n_hblk) + blockIdx.x % 8;
    if (w >= p.B * p.Hkv * p.n_split) return;
  }
  const int split = w % p.n_split;
  w /= p.n_split;
  const int g = w % p.Hkv;
  const int b = w / p.Hkv;

  // the row's position: the batch's, or (ragged batch) the row's own, which must lie in
  // [0, q_pos]; a position outside makes the row's partials NaN, so its out and lse are NaN.
  // Key ranges past a row's position are empty (m = -inf, l = 0, o = 0).
  int qp = p.q_pos;
  bool bad_pos = false;
  if (p.q_pos_rows != nullptr) {
    qp = p.q_pos_rows[b];
    bad_pos = qp < 0 || qp > p.q_pos;
    if (bad_pos) qp = 0;
  }
  const int key_end0 = qp + 1;  // keys 0 .. qp are visible
  const int h_begin = split * p.halves_per_split;
  const int h_end = min((key_end0 + 31) / 32, h_begin + p.halves_per_split);
  const int key_end = min(key_end0, 32 * h_end);  // first key past this split's range

  // Q^T operand: lane l holds head column l % 32 (zeros past the group), dimensions 16kk + 8hh
  // + e of this wave's k-steps, rotated at q_pos and scaled by log2(e)/sqrt(D).  Loaded before
  // the cache so that the rotation only waits for these loads.
  const int hc = hb * 32 + l32;  // head within the group
  const bool head_ok = hc < p.G;
  const int head = g * p.G + hc;
  // Lanes past the group load head 0 of the row (in bounds) and compute with it: every value a
  // lane holds belongs to its own head column, and those columns are never written.  The loads
  // are not consumed before the cache loads are issued, so the rotation's wait counts them
  // alone.
  u32x4 raw[NKW];
  {
    const int row_head = head_ok ? head : 0;
    if (tab.interleaved) {
      // adjacent-pair rotary form: dims 32kk + 16hh .. +15 (two 16-byte runs, split into evens
      // and odds after the cache loads are issued)
      const __bf16 *src = p.q + ((size_t)b * p.Hq + row_head) * D + 16 * hh;
#pragma unroll
      for (int j = 0; j < NKW / 2; ++j) {
        raw[j] = *reinterpret_cast<const u32x4 *>(src + 32 * kk_of(j));
        raw[j + NKW / 2] = *reinterpret_cast<const u32x4 *>(src + 32 * kk_of(j) + 8);
      }
    } else {
      const __bf16 *src = p.q + ((size_t)b * p.Hq + row_head) * D + 8 * hh;
#pragma unroll
      for (int j = 0; j < NKW; ++j) raw[j] = *reinterpret_cast<const u32x4 *>(src + 16 * kk_of(j));
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // the query loads go out before the cache's

  // The (b, g) run of tiles as buffer resources: a load whose (per-lane) offset lies past the
  // end returns zeros without a memory access, which is how the padded steps after h_end read
  // nothing.
  const uint32_t unit_bytes = (uint32_t)(p.S_pad / DBN) * TB;
  const size_t unit = (size_t)b * p.Hkv + g;
  const __amdgpu_buffer_rsrc_t kbuf = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(reinterpret_cast<const char *>(p.kr) + unit * unit_bytes), 0, (int)unit_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vbuf = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char *>(reinterpret_cast<const char *>(p.vt) + unit * unit_bytes), 0, (int)unit_bytes, 0x00020000);
  // half tile h = 2t + jb: keys 64t + 32jb .. +31.  K operand chunk kk: [chunk 2kk+hh][key][8];
  // V^T operand (tt, cb): key group 4jb + 2tt + hh, column 32cb + l32.
  const int k_lane = hh * 1024 + l32 * 16;
  const int v_lane = hh * 16 * D + l32 * 16 + wv * NCB * 512;
  auto half_base = [&](int h) __attribute__((always_inline)) {
    return h < h_end ? (h >> 1) * TB + (h & 1) * 512 : kPastEnd;
  };
  auto half_vbase = [&](int h) __attribute__((always_inline)) {
    return h < h_end ? (h >> 1) * TB + (h & 1) * 4 * 16 * D : kPastEnd;
  };
  bf16x8 kq[PD][NKW], vq[PD][2][NCB];
  auto load_half = [&](int h, int r) __attribute__((always_inline)) {
    const int kb = half_base(h), vb = half_vbase(h);
#pragma unroll
    for (int j = 0; j < NKW; ++j)
      kq[r][j] =
          __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kbuf, kb + k_lane + kk_of(j) * 2048, 0, 0));
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        vq[r][tt][cb] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vbuf, vb + v_lane + tt * 2 * 16 * D + cb * 512, 0, 0));
  };
  // The loop's first wait is shared by its entry and its back edge, so the entry issues the
  // half tiles in the loop's order, each behind a scheduling barrier: left to the scheduler,
  // half 0's first operand can be issued last, and that wait then drains every load.
#pragma unroll
  for (int r = 0; r < PD; ++r) {
    load_half(h_begin + r, r);
    __builtin_amdgcn_sched_barrier(0);
  }

  if (tab.interleaved) {
    // the evens are the reordered dims 16kk + 8hh + e, the odds D/2 + 16kk + 8hh + e
#pragma unroll
    for (int j = 0; j < NKW / 2; ++j) {
      const u32x4 lo = raw[j], hi = raw[j + NKW / 2];
      deinterleave16(lo, hi, raw[j], raw[j + NKW / 2]);
    }
  }
  bf16x8 qf[NKW];
#pragma unroll
  for (int j = 0; j < NKW / 2; ++j) {
    const int kk = kk_of(j);
    u32x4 olo, ohi;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      float r[2][2];
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const int e = 2 * ww + z;
        // both lane halves' frequencies at wave-uniform indices (scalar loads, which the
        // cache loads in flight do not hold up), then this lane's
        const double f0 = tab.rev[16 * kk + e], f1 = tab.rev[16 * kk + 8 + e];
        const float t = turn_fraction(qp, hh ? f1 : f0);
        const float sn = __builtin_amdgcn_sinf(t), cs = __builtin_amdgcn_cosf(t);  // turns
        const uint32_t lo = raw[j][ww], hi = raw[j + NKW / 2][ww];
        const float xv = z ? bf16_hi(lo) : bf16_lo(lo);
        const float yv = z ? bf16_hi(hi) : bf16_lo(hi);
        r[0][z] = (xv * cs - yv * sn) * p.q_scale;
        r[1][z] = (yv * cs + xv * sn) * p.q_scale;
      }
      olo[ww] = pack_bf16x2(r[0][0], r[0][1]);
      ohi[ww] = pack_bf16x2(r[1][0], r[1][1]);
    }
    qf[j] = __builtin_bit_cast(bf16x8, olo);
    qf[j + NKW / 2] = __builtin_bit_cast(bf16x8, ohi);
  }

  f32x16 o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{};
  float m_run = -INFINITY;  // running maximum of the base-2 scores of this lane's head
  float l_run = 0.f;        // this lane half's share of the running sum

  // Steps past h_end (padding to a multiple of PD) load zeros and have every key masked, so the
  // loop body needs no branch around its loads.  Both waves of a workgroup see the same key
  // range, so they meet at the same barriers.
  const int n_steps = (max(0, h_end - h_begin) + PD - 1) / PD * PD;
  for (int s0 = 0; s0 < n_steps; s0 += PD) {
#pragma unroll
    for (int r = 0; r < PD; ++r) {
      const int h = h_begin + s0 + r;
      f32x16 sc = f32x16{};
#pragma unroll
      for (int j = 0; j < NKW; ++j) sc = dec_mfma(kq[r][j], qf[j], sc);
      if constexpr (NW > 1) {
        // add the other wave's partial scores; the buffer alternates with the step, so a write
        // of the next step cannot overtake the other wave's read of this one (it has passed the
        // next barrier only after that read)
        const int buf = (s0 + r) & 1;
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          *reinterpret_cast<f32x4 *>(xs[buf][wv][v4][lane]) =
              f32x4{sc[4 * v4], sc[4 * v4 + 1], sc[4 * v4 + 2], sc[4 * v4 + 3]};
        __syncthreads();
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x4 t = *reinterpret_cast<const f32x4 *>(xs[buf][wv ^ 1][v4][lane]);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[4 * v4 + e] += t[e];
        }
      }
      // keys of this half: 32h + 8(v>>2) + 4hh + (v&3)
      if (32 * h + 31 >= key_end) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (32 * h + 8 * (v >> 2) + 4 * hh + (v & 3) >= key_end) sc[v] = -INFINITY;
        // The values of those keys are zeroed too: their weight is 0, but 0 times a NaN left in
        // the cache past a row's position (a ragged batch) would still be NaN.  Element e of the
        // V^T operand (tt, cb) is key swap23(8 qc + e) of the 64-key tile, qc = 4 jb + 2 tt + hh
        // its key chunk (swap23 exchanging bits 2 and 3, the accumulators' key order).
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int p0 = 8 * (4 * (h & 1) + 2 * tt + hh);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            u32x4 w = __builtin_bit_cast(u32x4, vq[r][tt][cb]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int pe = p0 + e;
              const int key = 64 * (h >> 1) + ((pe & ~12) | ((pe & 4) << 1) | ((pe & 8) >> 1));
              if (key >= key_end) w[e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
            }
            vq[r][tt][cb] = __builtin_bit_cast(bf16x8, w);
          }
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[v]);
      mx = dec_max_xor32(mx);
      // finite from the first step on: key 32 h_begin <= qp is in it (the loop runs only then)
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float rs = 0.f;
      bf16x8 pk[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        u32x4 wd;
#pragma unroll
        for (int ww = 0; ww < 4; ++ww) {
          const float e0 = __builtin_amdgcn_exp2f(sc[8 * tt + 2 * ww] - m_new);
          const float e1 = __builtin_amdgcn_exp2f(sc[8 * tt + 2 * ww + 1] - m_new);
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
        for (int cb = 0; cb < NCB; ++cb) o[cb] = dec_mfma(vq[r][tt][cb], pk[tt], o[cb]);
      load_half(h + PD, r);
    }
  }

  // partial result of this split for the heads of the group: o as [split][G heads][D] floats,
  // m and l per head
  if (head_ok) {
    const size_t prow = (unit * p.n_split + split) * p.G + hc;
    float *po = p.po + prow * D + wv * NCB * 32;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        *reinterpret_cast<f32x4 *>(po + 32 * cb + 8 * v4 + 4 * hh) =
            f32x4{o[cb][4 * v4], o[cb][4 * v4 + 1], o[cb][4 * v4 + 2], o[cb][4 * v4 + 3]};
  }
  const float l_tot = l_run + dec_xor32(l_run);
  if (wv == 0 && hh == 0 && head_ok) {  // both waves hold the same m and l
    const size_t prow = (unit * p.n_split + split) * p.G + hc;
    p.pm[prow] = bad_pos ? __builtin_nanf("") : m_run;
    p.pl[prow] = l_tot;
  }
}

// Joins the splits of every (b, head): m = max m_i, l = sum l_i 2^(m_i - m),
// out = sum o_i 2^(m_i - m) / l (bf16), lse = ln 2 * (m + log2 l).  One 256-thread workgroup
// per (b, head): R = 256 / (D/4) row groups of D/4 threads (16 bytes of a row each) take the
// splits sg, sg + R, ..., each group merging its rows with a running maximum, so that m, l and
// o of a row are loaded together (one trip to memory when n_split <= R); the R partial results
// are then joined by their maxima through LDS.
template <int D>
__global__ void __launch_bounds__(256) attn_decode_join_kernel(DecodeParams p) {
  constexpr int TPR = D / 4;      // threads per partial row
  constexpr int R = 256 / TPR;    // row groups
  __shared__ float red_m[R];
  __shared__ float red_l[R];
  __shared__ __attribute__((aligned(16))) float red_o[R][D];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;  // (b, head)
  const int head = bh % p.Hq;
  const int b = bh / p.Hq;
  const int g = head / p.G;
  const int hc = head % p.G;
  const size_t unit = (size_t)b * p.Hkv + g;
  auto row = [&](int s) __attribute__((always_inline)) { return (unit * p.n_split + s) * p.G + hc; };

  const int sg = tid / TPR;  // row group
  const int c4 = tid % TPR;  // dimensions 4 c4 .. 4 c4 + 3
  // A split past a ragged row's position is empty (m_i = -inf, l_i = 0, o_i = 0); split 0 never
  // is, so each row's final maximum is finite.  A group without rows, or with empty ones only,
  // keeps m = -inf and contributes 2^(-inf) = 0 below.  A factor whose maximum did not change is
  // 1 (also when both are -inf, where 2^(m - mn) would be NaN).
  float m = -INFINITY, l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = sg; s < p.n_split; s += R) {
    const size_t r = row(s);
    const float ms = p.pm[r], ls = p.pl[r];
    const f32x4 os = *reinterpret_cast<const f32x4 *>(p.po + r * D + 4 * c4);
    const float mn = fmaxf(m, ms);
    const float a = m == mn ? 1.f : __builtin_amdgcn_exp2f(m - mn);
    const float c = ms == mn ? 1.f : __builtin_amdgcn_exp2f(ms - mn);
    acc = acc * a + os * c;
    l = l * a + ls * c;
    m = mn;
  }
  *reinterpret_cast<f32x4 *>(&red_o[sg][4 * c4]) = acc;
  if (c4 == 0) {
    red_m[sg] = m;
    red_l[sg] = l;
  }
  __syncthreads();
  if (tid < D / 2) {
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < R; ++i) mt = fmaxf(mt, red_m[i]);
    float o0 = 0.f, o1 = 0.f, lt = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float c = __builtin_amdgcn_exp2f(red_m[i] - mt);
      o0 += red_o[i][2 * tid] * c;
      o1 += red_o[i][2 * tid + 1] * c;
      lt += red_l[i] * c;
    }
    const float inv = 1.0f / lt;
    *reinterpret_cast<uint32_t *>(p.out + ((size_t)b * p.Hq + head) * D + 2 * tid) = pack_bf16x2(o0 * inv, o1 * inv);
    if (tid == 0) p.lse[(size_t)b * p.Hq + head] = (mt + __log2f(lt)) * 0.69314718055994531f;
  }
}

template <int D>
hipError_t launch_decode(const DecodeParams &p, const RopeTable &tab, hipStream_t stream) {
  const long long ranges = (long long)p.B * p.Hkv * p.n_split;
  const long long wgs = p.n_hblk == 1 ? ranges : (ranges + 7) / 8 * 8 * p.n_hblk;
  hipLaunchKernelGGL((attn_decode_kernel<D, kDecodeDepth>), dim3((unsigned)wgs), dim3(D == 256 ? 128 : 64), 0, stream,
                     p, tab);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(attn_decode_join_kernel<D>, dim3((unsigned)((long long)p.B * p.Hq)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template hipError_t launch_decode<64>(const DecodeParams &, const RopeTable &, hipStream_t);
template hipError_t launch_decode<128>(const DecodeParams &, const RopeTable &, hipStream_t);
template hipError_t launch_decode<256>(const DecodeParams &, const RopeTable &, hipStream_t);

}  // namespace attn
