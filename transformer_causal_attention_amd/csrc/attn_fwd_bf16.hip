// Fused causal attention forward, bf16 in / bf16 out, fp32 accumulation, for gfx950.
//
// What is computed (per batch row b, query head h, query position i, K/V head g = h / G):
//   q' = RoPE(q_i) * log2(e)/sqrt(D)        (in registers, once per workgroup)
//   s_j = q' . k'_j                          (k' = RoPE(k), produced by the pre-pass)
//   online softmax over j <= i in base 2, out_i = sum_j p_j v_j / sum_j p_j,
//   lse_i = ln(2) * (max_j s_j + log2 sum_j 2^(s_j - max))
// Definitions: scores / sqrt(head_dim), mask of later keys, softmax over keys (llama3-from-
// scratch page: "attention score matrix", "causal mask", "softmax"); row max subtracted
// first (PaLM page, section 2.5); grouped K/V heads (llama3 page, "key-value sharing"); the
// IO-aware, tiled evaluation that never stores the score matrix is what the Picotron page
// calls flash attention ("Flash Attention integration and optimisation").
//
// Work decomposition.  A workgroup has 4 waves and owns one (batch, K/V head, block of
// query rows).  Each wave owns 32 query rows of one query head.  The hpw query heads of a
// workgroup (up to 4 of the G sharing the K/V head) all read the same staged K/V tiles, so
// grouped-query attention loads each tile once per hpw heads.  Row blocks are dispatched
// longest first (causal work grows with the row index) and consecutive workgroup ids walk
// the (batch, K/V head) units, which keeps one K/V head on one XCD's L2 when the number of
// units is a multiple of 8.
//
// Matrix layout.  With A = K tile (32 keys x 16 dims) and B = Q^T (16 dims x 32 rows), the
// 32x32x16 bf16 MFMA yields S^T: lane l holds query row l%32 and, in its 16 accumulators,
// keys 8*(v/4) + 4*(l/32) + v%4.  Row max and row sum are thus in-lane plus one exchange
// between the two lane halves.  O^T = V^T P^T uses those accumulators (packed to bf16) as
// its B operand unchanged; the key order they imply is matched by storing V transposed in
// LDS with key bits 2 and 3 swapped, so each lane fetches its A operand with one 16-byte
// read.  Keys above the diagonal are never loaded: the tile loop ends at the workgroup's
// last row, and a wave skips the 32-key blocks entirely above its own rows.

#include "attn_device.h"

namespace attn {

constexpr int BN = 64;      // keys per staged tile
constexpr int NWAVES = 4;   // waves per workgroup

template <int D>
struct Smem {
  static constexpr int KSTR = D * 2 + 16;   // bytes per staged key row (16 B pad: no bank conflicts)
  static constexpr int VSTR = BN * 2 + 16;  // bytes per transposed value row
  static constexpr int KBYTES = BN * KSTR;
  static constexpr int VBYTES = D * VSTR;
  static constexpr int BYTES = 2 * (KBYTES + VBYTES);  // double buffered
};

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Slot (8-byte unit) of key group jg (keys 4jg .. 4jg+3) inside a transposed value row:
// swap the two low bits of jg, then XOR-swizzle by the row's 8-column chunk.
__device__ __forceinline__ int v_slot(int jg, int c) {
  int s = (jg & ~3) | ((jg & 1) << 1) | ((jg >> 1) & 1);
  return s ^ (2 * ((c >> 3) & 7));
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) attn_fwd_bf16_kernel(FwdParams p, RopeTable tab) {
  constexpr int NKK = D / 16;   // MFMA steps over head_dim
  constexpr int NCB = D / 32;   // 32-column blocks of the output
  constexpr int KCH = D / 32;   // 16-byte key chunks per thread per tile
  using SM = Smem<D>;
  __shared__ __attribute__((aligned(16))) char smem[SM::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- work unit
  const int HG = p.G / p.hpw;
  const int u = blockIdx.x % p.n_units;
  const int rbo = blockIdx.x / p.n_units;
  const int rb = CAUSAL ? (p.n_row_blocks - 1 - rbo) : rbo;
  const int hg = u % HG;
  const int bg = u / HG;
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;
  const int rows_per_wg = 32 * (NWAVES / p.hpw);
  const int head = g * p.G + hg * p.hpw + (wave % p.hpw);
  const int row0 = rb * rows_per_wg + (wave / p.hpw) * 32;
  const int my_row = row0 + l32;
  const int S = p.S;
  const int kv_end = CAUSAL ? min(S, rb * rows_per_wg + rows_per_wg) : S;
  const int ntiles = (kv_end + BN - 1) / BN;
  // last 32-key block this wave needs (-1: the wave has no valid rows)
  const int kb_last = row0 >= S ? -1 : (CAUSAL ? min(row0 + 31, S - 1) : S - 1) / 32;

  // ---- Q prologue: load, rotate, fold the scale, convert to bf16 MFMA operands
  bf16x8 qf[NKK];
  {
    u32x4 raw[NKK];
    if (my_row < S) {
      const __bf16 *src = p.q + (((size_t)b * S + my_row) * p.Hq + head) * D + 8 * hh;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) raw[kk] = *reinterpret_cast<const u32x4 *>(src + 16 * kk);
    } else {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) raw[kk] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int kk = 0; kk < NKK / 2; ++kk) {
      u32x4 lo = raw[kk], hi = raw[kk + NKK / 2];
      u32x4 olo, ohi;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float r[2][2];
#pragma unroll
        for (int z = 0; z < 2; ++z) {
          const int e = 2 * w + z;  // column 16*kk + 8*hh + e, partner + D/2
          const double f = hh ? tab.rev[16 * kk + 8 + e] : tab.rev[16 * kk + e];
          const float t = turn_fraction(my_row, f);
          const float sn = __builtin_amdgcn_sinf(t);  // argument in turns
          const float cs = __builtin_amdgcn_cosf(t);
          const float x = z ? bf16_hi(lo[w]) : bf16_lo(lo[w]);
          const float y = z ? bf16_hi(hi[w]) : bf16_lo(hi[w]);
          r[0][z] = (x * cs - y * sn) * p.q_scale;
          r[1][z] = (y * cs + x * sn) * p.q_scale;
        }
        olo[w] = pack_bf16x2(r[0][0], r[0][1]);
        ohi[w] = pack_bf16x2(r[1][0], r[1][1]);
      }
      qf[kk] = __builtin_bit_cast(bf16x8, olo);
      qf[kk + NKK / 2] = __builtin_bit_cast(bf16x8, ohi);
    }
  }

  // ---- staging: K' tiles are contiguous (B, Hkv, S_pad, D); V is read from (B, S, Hkv, D)
  const __bf16 *kr_base = p.kr + ((size_t)b * p.Hkv + g) * (size_t)p.S_pad * D;
  const __bf16 *v_base = p.v + ((size_t)b * S * p.Hkv + g) * D;
  const size_t v_row_stride = (size_t)p.Hkv * D;
  // value staging item: 4 keys x 8 columns (D=64 uses only the first 128 threads)
  const bool v_stager = tid < 2 * D;
  const int v_cc = tid % (D / 8);
  const int v_jg = tid / (D / 8);

  u32x4 kreg[KCH];
  u32x4 vreg[4];

  auto load_tile = [&](int it) {
    const int kbase = it * BN;
    const __bf16 *ks = kr_base + (size_t)kbase * D;
#pragma unroll
    for (int r = 0; r < KCH; ++r) kreg[r] = *reinterpret_cast<const u32x4 *>(ks + (size_t)(tid + 256 * r) * 8);
    if (v_stager) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = kbase + 4 * v_jg + r;
        vreg[r] = j < S ? *reinterpret_cast<const u32x4 *>(v_base + (size_t)j * v_row_stride + 8 * v_cc)
                        : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  auto store_tile = [&](int buf) {
    char *kd = smem + buf * SM::KBYTES;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int id = tid + 256 * r;
      *reinterpret_cast<u32x4 *>(kd + (id / (D / 8)) * SM::KSTR + (id % (D / 8)) * 16) = kreg[r];
    }
    if (v_stager) {
      char *vd = smem + 2 * SM::KBYTES + buf * SM::VBYTES;
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int c = 8 * v_cc + x;
        const int y = x >> 1;
        const uint32_t sel = (x & 1) ? 0x07060302u : 0x05040100u;
        u32x2 w2;
        w2[0] = __builtin_amdgcn_perm(vreg[1][y], vreg[0][y], sel);
        w2[1] = __builtin_amdgcn_perm(vreg[3][y], vreg[2][y], sel);
        *reinterpret_cast<u32x2 *>(vd + c * SM::VSTR + 8 * v_slot(v_jg, c)) = w2;
      }
    }
  };

  float m_run = -INFINITY;  // running row max (base-2 scores)
  float l_run = 0.f;        // this lane half's share of the running row sum
  f32x16 o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) o[cb] = f32x16{};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const bool more = it + 1 < ntiles;
    if (more) load_tile(it + 1);

    const char *kd = smem + buf * SM::KBYTES;
    const char *vd = smem + 2 * SM::KBYTES + buf * SM::VBYTES;
    const int kbase = it * BN;

    // S^T = K' Q'^T for the tile's two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      if (2 * it + jb <= kb_last) {
        f32x16 acc = f32x16{};
        const char *ka = kd + (32 * jb + l32) * SM::KSTR + 16 * hh;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(ka + 32 * kk);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], acc, 0, 0, 0);
        }
        s[jb] = acc;
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[jb][v] = -INFINITY;
      }
    }

    // mask keys after the query (diagonal tile) and keys past the sequence end
    if ((CAUSAL && kbase + BN - 1 > row0) || kbase + BN > S) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int j = kbase + 32 * jb + 8 * (v >> 2) + 4 * hh + (v & 3);
          if ((CAUSAL && j > my_row) || j >= S) s[jb][v] = -INFINITY;
        }
    }

    // online softmax (base 2)
    float mx = s[0][0];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[jb][v]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // rows with no visible key yet
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float rsum = 0.f;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = __builtin_amdgcn_exp2f(s[jb][v] - m_use);
        s[jb][v] = e;
        rsum += e;
      }
    l_run = l_run * alpha + rsum;
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) o[cb] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      if (2 * it + jb <= kb_last) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          u32x4 pw;
#pragma unroll
          for (int w = 0; w < 4; ++w) pw[w] = pack_bf16x2(s[jb][8 * t + 2 * w], s[jb][8 * t + 2 * w + 1]);
          const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
          const int slot = 8 * jb + 4 * t + 2 * hh;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const int c = 32 * cb + l32;
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(vd + c * SM::VSTR + 8 * (slot ^ (2 * ((c >> 3) & 7))));
            o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[cb], 0, 0, 0);
          }
        }
      }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, store out (bf16) and lse (fp32, natural log)
  const float l_tot = l_run + xor32(l_run);
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
    if (hh == 0) p.lse[((size_t)b * p.Hq + head) * S + my_row] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_attn_bf16(const FwdParams &p, const RopeTable &tab, hipStream_t stream) {
  const long long blocks = (long long)p.n_units * p.n_row_blocks;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, stream, p, tab);
  return hipGetLastError();
}

template hipError_t launch_attn_bf16<64, true>(const FwdParams &, const RopeTable &, hipStream_t);
template hipError_t launch_attn_bf16<64, false>(const FwdParams &, const RopeTable &, hipStream_t);
template hipError_t launch_attn_bf16<128, true>(const FwdParams &, const RopeTable &, hipStream_t);
template hipError_t launch_attn_bf16<128, false>(const FwdParams &, const RopeTable &, hipStream_t);

}  // namespace attn
