// Fused causal attention forward for head_dim 256, bf16 in / bf16 out, fp32 accumulation, gfx950.
//
// Same definition as the head_dim 64 / 128 kernel (rotary embedding of q and k, scores divided
// by sqrt(head_dim), later keys masked, softmax with the row maximum subtracted, lse; Picotron,
// llama3-from-scratch and PaLM pages), for the head size of the PaLM page's largest model
// (section 3: 48 heads of 256, one shared K/V head).  At d = 256 the other kernel's staging (two
// wave groups, each with double-buffered 64-key K and V^T tiles in LDS, and 32 rows x d of
// accumulators per wave at two waves per SIMD) would need 256 KiB of LDS and more registers than
// two waves per SIMD have, so this kernel is built more simply:
//
//   - a workgroup is four waves, one per SIMD (two workgroups per CU: 64 KiB of LDS and at most
//     256 registers each), each owning 32 query rows of one head: hpw heads
//     of one K/V group times 4 / hpw row blocks, so every staged key serves four waves (heavy
//     row blocks are dispatched first, so the causal staircase fills the GPU evenly);
//   - the queries are loaded, rotated in registers and scaled by log2(e)/16 once;
//   - the prepared keys and values (the preparation pass's 64-key tiles: rotated K chunk-major,
//     V transposed) are copied 32 keys at a time from HBM/L2 straight into LDS (double
//     buffered, the next half's copy running while the current one is used), and every MFMA
//     operand is one 16-byte LDS read;
//   - S^T = K Q^T and O^T = V^T P^T on the 32x32x16 bf16 MFMA (the accumulator layouts of the
//     decode kernel), a running maximum per 32 keys that moves only when it grows by more than
//     2^8, and the rescale of o and l only then.
//
// Keys above the diagonal are never loaded.  Rows with no visible key (only in a shard of later
// keys) give out 0 and lse -inf.

#include <hip/hip_ext.h>

#include "attn_device.h"

namespace attn {

typedef __attribute__((address_space(3))) void *LDS_PTR;

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
__global__ void __launch_bounds__(256, 2) attn_fwd_d256_kernel(FwdParams p, RopeTable tab) {
  constexpr int D = 256;
  constexpr int NKK = D / 16;     // MFMA steps over head_dim
  constexpr int NCB = D / 32;     // 32-column blocks of the output
  constexpr int TB = 64 * D * 2;  // bytes of one prepared 64-key tile
  constexpr int HB = 32 * D * 2;  // bytes of one staged 32-key half (K or V^T)
  // staged halves, double buffered: K as [32 dim chunks][32 keys][8], V^T as [4 key chunks][D][8]
  __shared__ __attribute__((aligned(1024))) char ldsk[2][HB];
  __shared__ __attribute__((aligned(1024))) char ldsv[2][HB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // workgroup -> (b, K/V head g, head group, row block), heaviest row blocks first.  The four
  // waves cover hpw heads x (4 / hpw) sub-blocks of 32 rows and share every staged half.
  const int nrb = p.n_row_blocks;
  const int RPB = p.rows_per_blk;
  int w = blockIdx.x;
  const int rb = nrb - 1 - w % nrb;
  w /= nrb;
  const int HG = p.G / p.hpw;
  const int hg = w % HG;
  w /= HG;
  const int g = w % p.Hkv;
  const int b = w / p.Hkv;
  const int head = g * p.G + hg * p.hpw + wave % p.hpw;
  const int S = p.S;
  const int delta = p.delta;
  const int row0 = rb * RPB + (wave / p.hpw) * 32;
  const int my_row = row0 + l32;
  // keys the workgroup needs: query i sees key j iff j <= i + delta (causal), j < S
  const int kend = CAUSAL ? max(0, min(S, min(S, (rb + 1) * RPB) + delta)) : S;
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
  // Copy of 32-key half h (keys 32h .. 32h+31: tile h/2, half h%2) into buffer h%2, 16 bytes per
  // lane per instruction, global -> LDS with no registers; each wave issues 4 of the 16 K and 4
  // of the 16 V^T instructions.
  //   K: instruction ii moves dim chunks 2ii (lanes 0-31) and 2ii+1 (lanes 32-63), keys l32:
  //      global (2ii + hh) * 1024 + (32(h%2) + l32) * 16 -> LDS ii * 1024 + lane * 16
  //   V^T: the half's 4 key chunks are one contiguous 16 KiB run: global 4(h%2) * 16D + ii * 1024
  //      + lane * 16 -> LDS ii * 1024 + lane * 16
  const uint32_t k_voff = (uint32_t)(hh * 1024 + l32 * 16);
  const uint32_t v_voff = (uint32_t)(lane * 16);
  auto stage = [&](int h) __attribute__((always_inline)) {
    char *kd = ldsk[h & 1];
    char *vd = ldsv[h & 1];
    const uint32_t tile = (uint32_t)(h >> 1) * TB;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ii = wave * 4 + r;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kbuf, (LDS_PTR)(kd + ii * 1024), 16, k_voff,
                                               tile + (uint32_t)(h & 1) * 512 + (uint32_t)ii * 2048, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vbuf, (LDS_PTR)(vd + ii * 1024), 16, v_voff,
                                               tile + (uint32_t)(h & 1) * 4 * 16 * D + (uint32_t)ii * 1024, 0, 0);
    }
  };
  if (n_halves > 0) stage(0);

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
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  f32x16 o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{};
  float m_run = -INFINITY;  // running maximum of this row's base-2 scores
  float l_run = 0.f;        // this lane half's share of the running sum

  for (int h = 0; h < n_halves; ++h) {
    // the next half goes into the other buffer, which every wave finished reading before the
    // barrier that ended the previous step
    if (h + 1 < n_halves) stage(h + 1);
    const char *kd = ldsk[h & 1];
    const char *vd = ldsv[h & 1];
    // S^T = K Q^T: K operand = dim chunk 2kk + hh, key l32 of the staged half
    f32x16 sc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      sc = d256_mfma(*reinterpret_cast<const bf16x8 *>(kd + (2 * kk + hh) * 512 + l32 * 16), qf[kk], sc);
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
    // The reference m moves only when a row's maximum passes it by more than 8 (base 2), and
    // then to that maximum: the probabilities stay at most 2^8, and o and l are rescaled only in
    // steps where some row of the wave moved.  A row's first visible key always moves it, so the
    // first maximum is exact.
    const bool grow = mx > m_run + 8.f;  // false while the row has seen no key
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;  // exp2(-inf) = 0 on a fresh row
      m_run = grow ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;  // a row with no visible key yet
    // l sums the probabilities as rounded to bf16 for the P.V product, so the weights that
    // multiply V are exactly normalised by l
    float rs = 0.f;
    bf16x8 pk[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      u32x4 wd;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float e0 = __builtin_amdgcn_exp2f(sc[8 * tt + 2 * ww] - m_use);
        const float e1 = __builtin_amdgcn_exp2f(sc[8 * tt + 2 * ww + 1] - m_use);
        const uint32_t pw = pack_bf16x2(e0, e1);
        rs += bf16_lo(pw) + bf16_hi(pw);
        wd[ww] = pw;
      }
      pk[tt] = __builtin_bit_cast(bf16x8, wd);
    }
    l_run += rs;
    // O^T += V^T P^T: V^T operand = key chunk 2tt + hh of the half, column 32cb + l32
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
        o[cb] = d256_mfma(*reinterpret_cast<const bf16x8 *>(vd + (2 * tt + hh) * 16 * D + (32 * cb + l32) * 16),
                          pk[tt], o[cb]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
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
  const long long blocks = (long long)p.n_units * p.n_row_blocks;
  hipExtLaunchKernelGGL((attn_fwd_d256_kernel<CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, stream, ev_start,
                        ev_stop, 0, p, tab);
  return hipGetLastError();
}

template hipError_t launch_attn_d256<true>(const FwdParams &, const RopeTable &, hipStream_t, hipEvent_t, hipEvent_t);
template hipError_t launch_attn_d256<false>(const FwdParams &, const RopeTable &, hipStream_t, hipEvent_t, hipEvent_t);

}  // namespace attn
