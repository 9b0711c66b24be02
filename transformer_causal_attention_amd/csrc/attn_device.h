// Device-side types and helpers shared by the attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace attn {

constexpr int kMaxHalfDim = 128;  // head_dim <= 256

// Rotary frequencies in revolutions per position: rope_theta^(-2i/d) / (2*pi), i < d/2.
// Computed on the host in double precision and passed by value, so every index used by
// the kernels is a compile-time constant or wave-uniform (scalar loads, no scratch).
//
// interleaved = 1 selects the adjacent-pair rotary form, where dims (2i, 2i+1) turn together by
// frequency i (llama3-from-scratch page, the rotary embedding taken as complex numbers) instead
// of (i, i + d/2).  It equals the half-split rotation applied to the head dims reordered as
// (x0, x2, .., x_{d-2}, x1, x3, .., x_{d-1}); q and k are reordered alike, so their dot products
// are unchanged, and the kernels simply read q and k in that order (and write dq, dk back in the
// original one).  V and the output are not reordered.
struct RopeTable {
  double rev[kMaxHalfDim];
  int interleaved;
};

// 16 consecutive bf16 values (lo = elements 0..7, hi = 8..15) split into the even-indexed
// ones (ev) and the odd-indexed ones (od), each in order: the reordering of the adjacent-pair
// rotary form.
__device__ __forceinline__ void deinterleave16(const u32x4 &lo, const u32x4 &hi, u32x4 &ev, u32x4 &od) {
  u32x4 e, o;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = w < 2 ? lo[2 * w] : hi[2 * w - 4];
    const uint32_t y = w < 2 ? lo[2 * w + 1] : hi[2 * w - 3];
    e[w] = (x & 0xffffu) | (y << 16);
    o[w] = (x >> 16) | (y & 0xffff0000u);
  }
  ev = e;
  od = o;
}

// Position in the original head dims of reordered dim c (see RopeTable).
__device__ __forceinline__ int rope_src_dim(int c, int half, int interleaved) {
  return interleaved ? (c < half ? 2 * c : 2 * (c - half) + 1) : c;
}

// Everything the bf16 attention kernel needs besides the rotation table.
struct FwdParams {
  const __bf16 *q;   // (B, S, Hq, D)
  const __bf16 *kr;  // rotated keys, 64-key tiles (B, Hkv, S_pad/64) x [D/8][64][8]
  const __bf16 *vt;  // transposed values, 64-key tiles (B, Hkv, S_pad/64) x [8][D][8]
  __bf16 *out;       // (B, S, Hq, D)
  float *lse;        // (B, Hq, S)
  int B, S, Hq, Hkv, G, S_pad;
  int hpw;           // query heads per wave group (1, 2 or 4)
  int rows_per_blk;  // query rows per row block: 32 * (4 / hpw)
  int n_units;       // B * Hkv * (G / hpw)
  int n_row_blocks;  // ceil(S / rows_per_blk)
  int n_pairs;       // ceil(n_row_blocks / 2): workgroups per unit
  int q_pos0;        // position of query row 0 (a sequence shard's offset; 0 otherwise)
  int delta;         // q_pos0 - k_pos0: key j is visible to query i iff j <= i + delta (causal)
  float q_scale;     // log2(e) / sqrt(D): scores come out in the base-2 domain
  int dual;          // head_dim 64: each workgroup runs two units (one per wave group)
  // One-launch form: the attention kernel prepares the tiles itself (each wave group
  // rotates the keys or transposes the values of some 64-key tiles, publishes a flag per
  // tile half, then waits for the flags of every tile it reads).
  const __bf16 *k;   // (B, S, Hkv, D) as given
  const __bf16 *v;   // (B, S, Hkv, D) as given
  unsigned long long *flags;  // (B, Hkv, S_pad/64, 2): tag of the call that wrote each half
  unsigned int *status;       // set to kStatusTimeout by a workgroup whose wait ran out
  unsigned long long tag;     // this call's tag (never a value an earlier call left behind)
  unsigned long long await_tag;  // the tag the waits look for: tag (or, to test the bounded
                                 // wait, a value no workgroup writes)
  int max_polls;     // bound of each wait, in polls
  int k_pos0;        // position of key row 0
  int prep_workers;  // wave groups that prepare tiles of one (b, K/V head)
  int prep_rounds;   // jobs per wave group, rounded up: ceil(2 * S_pad/64 / prep_workers)
};

// Value left in FwdParams::status when a workgroup gave up waiting for a tile (its rows are
// then written as NaN).
constexpr unsigned int kStatusTimeout = 1u;

struct F32Params {
  const float *q, *k, *v;
  float *out;
  float *lse;
  int B, S, Hq, Hkv, G;
  int n_row_blocks;
  int q_pos0, k_pos0;  // positions of query row 0 and key row 0
  float q_scale;
};

struct PrepParams {
  const __bf16 *k;  // (B, S, Hkv, D)
  const __bf16 *v;  // (B, S, Hkv, D)
  __bf16 *kr;       // 64-key tiles (B, Hkv, S_pad/64) x [D/8][64][8]
  __bf16 *vt;       // 64-key tiles (B, Hkv, S_pad/64) x [8][D][8]
  int B, S, Hkv, S_pad;  // S: rows that hold keys (later rows of a tile are zeros);
                         // S_pad: keys per (b, g) in the output layout, a multiple of 64
  int S_rows;            // rows per batch row in k and v (their batch stride), >= S
  int tile0, n_run;      // the tiles prepared: [tile0, tile0 + n_run)
  int k_pos0;            // position of key row 0
};

// Merge of two partial results: o1, o2, out (B, S, H, D) of the element type; lse1, lse2, lse
// (B, H, S) float32.  out / lse may be o1 / lse1 or o2 / lse2.
struct MergeParams {
  const void *o1, *o2;
  const float *lse1, *lse2;
  void *out;
  float *lse;
  long long rows;  // B * S * H
  int S, H;
};

// Decode step: one query row per (b, head) at position q_pos against a prepared K/V cache.
struct DecodeParams {
  const __bf16 *q;   // (B, Hq, D)
  const __bf16 *kr;  // prepared cache: rotated keys, 64-key tiles (B, Hkv, S_pad/64) x [D/8][64][8]
  const __bf16 *vt;  // prepared cache: transposed values, (B, Hkv, S_pad/64) x [8][D][8]
  __bf16 *out;       // (B, Hq, D)
  float *lse;        // (B, Hq)
  float *po;         // partial outputs: (B, Hkv, n_split, G, D)
  float *pm, *pl;    // partial maxima and sums: (B, Hkv, n_split, G)
  int B, Hq, Hkv, G, S_pad;
  int q_pos;             // the query's position (keys 0 .. q_pos are visible); with q_pos_rows,
                         // the largest position any batch row may have (it sizes the key splits)
  const int *q_pos_rows; // nullptr, or each batch row's own position (B entries, device)
  int n_hblk;            // blocks of 32 heads per K/V head: ceil(G / 32)
  int n_split;           // key ranges per (b, K/V head)
  int halves_per_split;  // 32-key half tiles per key range
  float q_scale;
};

// Backward pass: 32-row blocks of queries and keys, operands pre-laid-out per block.
//   "c" layout (chunk-major), one 32-row block: [D/8 chunks][32 rows][8 dims]
//   "t" layout (transposed), one 32-row block: [2 halves][2][D columns][8 rows], where row
//     16*half + swap23(8*j + e) sits at (half, j, column, e), swap23 exchanging bits 2 and 3
struct BwdParams {
  const __bf16 *q, *k, *v;  // (B, S, Hq | Hkv, D)
  const __bf16 *out, *dout; // (B, S, Hq, D)
  const float *lse;         // (B, Hq, S)
  __bf16 *dq, *dk, *dv;     // like q, k, v
  // workspace, one T = 32*D*2-byte tile per (b, head, block)
  __bf16 *kc, *kt, *vc;     // (B, Hkv, NB) tiles: rotated keys (c, t), values (c)
  __bf16 *qc, *qt, *dc, *dt;  // (B, Hq, NB) tiles: rotated q * log2(e)/sqrt(D) (c), rotated
                              // q / sqrt(D) (t), dout (c, t)
  float *l2, *dd;           // (B, Hq, NB*32): lse * log2(e) (+inf past S); rowsum(dout * out)
  int B, S, Hq, Hkv, G, NB, n_pairs, W, causal;
  // head splits of the dk/dv kernels: the HS workgroups of a (b, g, key-block group) take the
  // group's query heads hs, hs + HS, ... (head_dim 64, 128; head_dim 256 and the per-head
  // kernel: passes hs, hs + HS, ... of W heads) and, when HS > 1, leave fp32 partial sums in
  // part ([2][HS][B*Hkv][NB*32][D]: dk' before its rotation back, then dv), which a reduction
  // kernel adds up (in hs order) and writes
  int HS;
  float *part;
  int q_pos0, k_pos0;       // positions of query row 0 and key row 0 (a sequence shard's offsets)
  float scale_log2;         // log2(e) / sqrt(D)
  float inv_sqrt_d;         // 1 / sqrt(D)
};

// Fraction of a turn for position p and frequency f (revolutions per position):
// p * f is formed in double precision and reduced to [-0.5, 0.5], so the angle stays
// accurate to ~1e-12 turns even at p = 32767, where a float product would be off by
// ~1e-3 rad.
__device__ __forceinline__ float turn_fraction(int p, double f) {
  double r = (double)p * f;
  return (float)(r - __builtin_rint(r));
}

// Accurate sin/cos of 2*pi*t for t in [-0.5, 0.5] (library sincospi).
__device__ __forceinline__ void sincos_turns(float t, float *s, float *c) {
  sincospif(2.0f * t, s, c);
}

// One rotary pair (x, y) turned by the angle with cosine c and sine s: (x c - y s, y c + x s),
// each with one explicit fused multiply-add so that every kernel that prepares keys rounds
// alike.
__device__ __forceinline__ void rotate_pair(float x, float y, float c, float s, float &rx, float &ry) {
  rx = __builtin_fmaf(x, c, -(y * s));
  ry = __builtin_fmaf(y, c, x * s);
}

// Two rotary pairs, (x0, y0) and (x1, y1) unpacked from the bf16 words xw = (x0, x1) and
// yw = (y0, y1), turned by (c0, s0) and (c1, s1); returns the packed bf16 words (x0', x1') and
// (y0', y1').
__device__ __forceinline__ u32x2 rotate_packed(uint32_t xw, uint32_t yw, float c0, float s0, float c1, float s1);

// Raw (unformatted, byte-addressed) buffer resource over `bytes` bytes at `base`.  A buffer load
// takes its base from scalar registers and a 32-bit offset per lane from one VGPR.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ u32x2 rotate_packed(uint32_t xw, uint32_t yw, float c0, float s0, float c1, float s1) {
  float a0, b0, a1, b1;
  rotate_pair(bf16_lo(xw), bf16_lo(yw), c0, s0, a0, b0);
  rotate_pair(bf16_hi(xw), bf16_hi(yw), c1, s1, a1, b1);
  return u32x2{pack_bf16x2(a0, a1), pack_bf16x2(b0, b1)};
}

}  // namespace attn
