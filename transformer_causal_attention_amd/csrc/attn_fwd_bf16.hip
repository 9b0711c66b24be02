// Fused causal attention forward, bf16 in / bf16 out, fp32 accumulation, for gfx950.
//
// What is computed (per batch row b, query head h, query position i, K/V head g = h / G):
//   q' = RoPE(q_i) * log2(e)/sqrt(D)        (in registers, once per row block)
//   s_j = q' . k'_j                          (k' = RoPE(k), produced by the pre-pass)
//   online softmax over j <= i in base 2, out_i = sum_j p_j v_j / sum_j p_j,
//   lse_i = ln(2) * (max_j s_j + log2 sum_j 2^(s_j - max))
// Definitions: scores / sqrt(head_dim), mask of later keys, softmax over keys (llama3-from-
// scratch page: "attention score matrix", "causal mask", "softmax"); row max subtracted
// first (PaLM page, section 2.5); grouped K/V heads (llama3 page, "key-value sharing"); the
// IO-aware, tiled evaluation that never stores the score matrix is what the Picotron page
// calls flash attention ("Flash Attention integration and optimisation").
//
// Work decomposition.  A workgroup has 8 waves in two groups of 4 (wave w runs on SIMD w%4,
// so every SIMD holds one wave of each group).  In a group each wave owns 32 query rows of
// one query head; the hpw heads of the group (up to 4 of the G sharing the K/V head) read
// the same K/V tiles, so grouped-query attention stages each tile once per hpw heads.
// Causal work grows linearly with the row block, so a workgroup takes the pair of row blocks
// (r, n-1-r): group A runs all of block r plus the first x key tiles of block n-1-r, group B
// the remaining key tiles of block n-1-r, with x chosen so both groups run the same number of
// tiles; A then hands its partial (max, sum, accumulator) for block n-1-r to B through LDS and
// B merges the two (the same logsumexp merge that joins sequence shards).  Every workgroup
// therefore does the same work, and consecutive workgroup ids walk the (batch, K/V head)
// units so one K/V head stays on one XCD's L2 when the unit count is a multiple of 8.
//
// Data movement.  K' and V tiles (64 keys) go from HBM straight into LDS (global_load_lds,
// 16 bytes per lane, no registers), double buffered per group, with XOR swizzles of the
// 16-byte chunks so the MFMA operand reads below are free of bank conflicts.
//
// Matrix layout.  With A = K tile (32 keys x 16 dims) and B = Q^T (16 dims x 32 rows), the
// 32x32x16 bf16 MFMA yields S^T: lane l holds query row l%32 and, in its 16 accumulators,
// keys 8*(v/4) + 4*(l/32) + v%4.  Row max and row sum are thus in-lane plus one exchange
// between the lane halves.  O^T = V^T P^T takes those accumulators (packed to bf16) as its B
// operand unchanged; the matching A operand (V^T, keys along k in that order) is fetched from
// the row-major V tile with the transposing LDS read ds_read_tr16_b64.  Keys above the
// diagonal are never loaded, and a wave skips the 32-key blocks entirely above its rows.
// The accumulator is rescaled only when a row maximum grows by more than 2^8 (a wave-uniform
// test): probabilities are then taken against a stale maximum and stay below 256, which
// bf16 and fp32 hold exactly as well as values below 1.

#include "attn_device.h"

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

namespace attn {

constexpr int BN = 64;  // keys per staged tile
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));

__device__ __forceinline__ float xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0] holds lane l%32's value in every lane, r[1] lane 32 + l%32's
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 16-byte-chunk swizzles (chunk index XOR f(row)) of the staged tiles.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 15) : ((row ^ (row >> 3)) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  const int a = row & 3;
  return D == 128 ? (4 * a + 2 * (a >> 1)) : 2 * a;
}

// Each lane copies 16 bytes from `g` to lds_base + 16 * lane (lds_base is wave-uniform).
__device__ __forceinline__ void lds_dma16(const void *g, char *lds_base) {
  __builtin_amdgcn_global_load_lds((GLB_AS void *)g, (LDS_AS void *)lds_base, 16, 0, 0);
}

__device__ __forceinline__ u32x2 lds_read_tr16(const char *p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)p);
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512) attn_fwd_bf16_kernel(FwdParams p, RopeTable tab) {
  constexpr int NKK = D / 16;      // MFMA steps over head_dim
  constexpr int NCB = D / 32;      // 32-column blocks of the output
  constexpr int TB = BN * D * 2;   // bytes of one staged K or V tile
  constexpr int RB = 2 * D;        // bytes per tile row
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int DMA_PER_WAVE = TB / 4096;  // 1 KiB copies per wave per tile (4 waves per group)
  // [group][buffer][K, V]
  __shared__ __attribute__((aligned(1024))) char smem[8 * TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep in SGPRs
  const int grp = wave >> 2;
  const int gw = wave & 3;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work: unit (b, g, head group) and row-block pair
  const int HG = p.G / p.hpw;
  const int u = blockIdx.x % p.n_units;
  const int pi = blockIdx.x / p.n_units;
  const int hg = u % HG;
  const int bg = u / HG;
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;
  const int S = p.S;
  const int RPB = p.rows_per_blk;
  const int r_lo = pi;
  const int r_hi = p.n_row_blocks - 1 - pi;
  const int t_lo = ((CAUSAL ? min(S, (r_lo + 1) * RPB) : S) + BN - 1) / BN;
  const int t_hi = ((CAUSAL ? min(S, (r_hi + 1) * RPB) : S) + BN - 1) / BN;
  const bool two = r_lo != r_hi;
  const int x = two ? (t_hi - t_lo) / 2 : t_hi / 2;  // key tiles of block r_hi run by group A
  // group A: segment 0 = (r_lo, tiles [0, t_lo)) when two, then segment 1 = (r_hi, [0, x));
  // group B: segment 1 = (r_hi, [x, t_hi)).
  const int len0 = (grp == 0 && two) ? t_lo : 0;
  const int k1s = grp == 0 ? 0 : x;
  const int n_mine = len0 + (grp == 0 ? x : t_hi - x);
  const int n_iter = max((two ? t_lo : 0) + x, t_hi - x);

  const int head = g * p.G + hg * p.hpw + (gw % p.hpw);
  const int sub = gw / p.hpw;

  const __bf16 *kr_base = p.kr + ((size_t)b * p.Hkv + g) * (size_t)p.S_pad * D;
  const __bf16 *v_base = p.v + ((size_t)b * S * p.Hkv + g) * D;
  const size_t v_rs = (size_t)p.Hkv * D;

  // per-lane operand offsets (loop invariant)
  const int k_sw = k_swz<D>(l32);
  const int sig = lane & 15;
  const int v_row = 4 * hh + (sig >> 2);                       // + 32jb + 16t + 8e2
  const int v_ch = 2 * ((lane >> 4) & 1) + ((sig & 3) >> 1);   // + 4cb
  const int v_sw = v_swz<D>(sig >> 2);
  const int v_half = 8 * (sig & 1);

  auto stage = [&](int i, int buf) {
    const int kt = i < len0 ? i : k1s + (i - len0);
    char *kd = smem + ((grp * 2 + buf) * 2 + 0) * TB;
    char *vd = smem + ((grp * 2 + buf) * 2 + 1) * TB;
    const __bf16 *ks = kr_base + (size_t)kt * BN * D;
#pragma unroll
    for (int r = 0; r < DMA_PER_WAVE; ++r) {
      const int blk = gw * DMA_PER_WAVE + r;
      const int L = blk * 64 + lane;  // 16-byte chunk of the tile this lane fills
      const int row = L / CPR;
      const int ch = L % CPR;
      lds_dma16(ks + row * D + 8 * (ch ^ k_swz<D>(row)), kd + blk * 1024);
      const int j = min(kt * BN + row, S - 1);  // rows past S are masked; any finite value works
      lds_dma16(v_base + (size_t)j * v_rs + 8 * (ch ^ v_swz<D>(row)), vd + blk * 1024);
    }
  };

  bf16x8 qf[NKK];
  float m_run = -INFINITY;  // running row max (base-2 scores), stale by at most 8
  float l_run = 0.f;        // this lane half's share of the running row sum
  f32x16 o[NCB];
  int row0 = 0, kb_last = -1, cur_seg = -1;

  auto begin_seg = [&](int seg) {
    const int R = seg == 0 ? r_lo : r_hi;
    row0 = R * RPB + sub * 32;
    kb_last = row0 >= S ? -1 : (CAUSAL ? min(row0 + 31, S - 1) : S - 1) / 32;
    const int my_row = row0 + l32;
    u32x4 raw[NKK];
    if (my_row < S) {
      const __bf16 *src = p.q + (((size_t)b * S + my_row) * p.Hq + head) * D + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) raw[kk] = *reinterpret_cast<const u32x4 *>(src + 16 * kk);
    } else {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) raw[kk] = u32x4{0u, 0u, 0u, 0u};
    }
    // rotate pairs (c, c + D/2): lane holds columns 16kk + 8hh + e in raw[kk], kk < NKK/2
#pragma unroll
    for (int kk = 0; kk < NKK / 2; ++kk) {
      u32x4 olo, ohi;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float r[2][2];
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const int e = 2 * w + z;
          const double f = hh ? tab.rev[16 * kk + 8 + e] : tab.rev[16 * kk + e];
          const float t = turn_fraction(my_row, f);
          const float sn = __builtin_amdgcn_sinf(t);  // argument in turns
          const float cs = __builtin_amdgcn_cosf(t);
          const uint32_t lo = raw[kk][w], hi = raw[kk + NKK / 2][w];
          const float xv = z ? bf16_hi(lo) : bf16_lo(lo);
          const float yv = z ? bf16_hi(hi) : bf16_lo(hi);
          r[0][z] = (xv * cs - yv * sn) * p.q_scale;
          r[1][z] = (yv * cs + xv * sn) * p.q_scale;
        }
        olo[w] = pack_bf16x2(r[0][0], r[0][1]);
        ohi[w] = pack_bf16x2(r[1][0], r[1][1]);
      }
      qf[kk] = __builtin_bit_cast(bf16x8, olo);
      qf[kk + NKK / 2] = __builtin_bit_cast(bf16x8, ohi);
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{};
  };

  auto store_seg = [&]() {
    const float l_tot = l_run + xor32(l_run);
    const int my_row = row0 + l32;
    if (my_row < S) {
      const float inv = 1.0f / l_tot;
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
        p.lse[((size_t)b * p.Hq + head) * S + my_row] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
    }
  };

  auto compute_tile = [&](int kt, int buf) {
    const char *kd = smem + ((grp * 2 + buf) * 2 + 0) * TB;
    const char *vd = smem + ((grp * 2 + buf) * 2 + 1) * TB;
    const int kbase = kt * BN;
    f32x16 s[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      if (2 * kt + jb <= kb_last) {
        f32x16 acc = f32x16{};
        const int row = 32 * jb + l32;
        const int sw = D == 128 ? k_sw : k_swz<D>(row);
        const char *ka = kd + row * RB;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ka + 16 * ((2 * kk + hh) ^ sw));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], acc, 0, 0, 0);
        }
        s[jb] = acc;
      }
    }
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      if (2 * kt + jb > kb_last) continue;  // wave-uniform
      const int kb0 = kbase + 32 * jb;
      if ((CAUSAL && kb0 + 31 > row0) || kb0 + 32 > S) {
        const int my_row = row0 + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = kb0 + 8 * (v >> 2) + 4 * hh + (v & 3);
          if ((CAUSAL && j > my_row) || j >= S) s[jb][v] = -INFINITY;
        }
      }
      float mx = s[jb][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[jb][v]);
      mx = max_xor32(mx);
      // every row of a processed block has a visible key, so mx is finite here
      if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
        m_run = m_new;
      }
      float rsum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = __builtin_amdgcn_exp2f(s[jb][v] - m_run);
        s[jb][v] = e;
        rsum += e;
      }
      l_run += rsum;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 pw;
#pragma unroll
        for (int w = 0; w < 4; ++w) pw[w] = pack_bf16x2(s[jb][8 * t + 2 * w], s[jb][8 * t + 2 * w + 1]);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        const char *vr = vd + (32 * jb + 16 * t + v_row) * RB + v_half;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const int ch = (4 * cb + v_ch) ^ v_sw;
          const u32x2 a0 = lds_read_tr16(vr + 16 * ch);
          const u32x2 a1 = lds_read_tr16(vr + 8 * RB + 16 * ch);
          const u32x4 a4 = {a0[0], a0[1], a1[0], a1[1]};
          o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4), pb, o[cb], 0, 0, 0);
        }
      }
    }
  };

  // ---- main loop: both groups step through their tile lists in lockstep
  if (n_mine > 0) stage(0, 0);
  wait_vm_all();
  __syncthreads();
  for (int i = 0; i < n_iter; ++i) {
    const int buf = i & 1;
    if (i + 1 < n_mine) stage(i + 1, buf ^ 1);
    if (i < n_mine) {
      const int seg = i < len0 ? 0 : 1;
      if (seg != cur_seg) {
        if (cur_seg == 0) store_seg();
        begin_seg(seg);
        cur_seg = seg;
      }
      compute_tile(i < len0 ? i : k1s + (i - len0), buf);
    }
    wait_vm_all();
    __syncthreads();
  }

  // ---- finish: A stores block r_lo if it still holds it; the split block is merged in B
  if (grp == 0 && cur_seg == 0) store_seg();
  if (x > 0) {
    float *mo = reinterpret_cast<float *>(smem);  // tile buffers are free after the last barrier
    float *mm = mo + 4 * NCB * 16 * 64;
    if (grp == 0) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mo[((gw * NCB + cb) * 16 + v) * 64 + lane] = o[cb][v];
      mm[gw * 64 + lane] = m_run;
      mm[256 + gw * 64 + lane] = l_run;
    }
    __syncthreads();
    if (grp == 1) {
      const float ma = mm[gw * 64 + lane];
      const float la = mm[256 + gw * 64 + lane];
      const float m_new = fmaxf(ma, m_run);  // finite for every row below S
      const float ca = __builtin_amdgcn_exp2f(ma - m_new);
      const float cb_ = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run = la * ca + l_run * cb_;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[cb][v] = mo[((gw * NCB + cb) * 16 + v) * 64 + lane] * ca + o[cb][v] * cb_;
      m_run = m_new;
    }
  }
  if (grp == 1) store_seg();
}

template <int D, bool CAUSAL>
hipError_t launch_attn_bf16(const FwdParams &p, const RopeTable &tab, hipStream_t stream) {
  const long long blocks = (long long)p.n_units * p.n_pairs;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(512), 0, stream, p, tab);
  return hipGetLastError();
}

template hipError_t launch_attn_bf16<64, true>(const FwdParams &, const RopeTable &, hipStream_t);
template hipError_t launch_attn_bf16<64, false>(const FwdParams &, const RopeTable &, hipStream_t);
template hipError_t launch_attn_bf16<128, true>(const FwdParams &, const RopeTable &, hipStream_t);
template hipError_t launch_attn_bf16<128, false>(const FwdParams &, const RopeTable &, hipStream_t);

}  // namespace attn
