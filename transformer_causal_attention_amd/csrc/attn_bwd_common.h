// Helpers shared by the backward kernels' sources: operand loads, the MFMA, the result
// layout, the workgroup order and the rotation of a row of 8 values.
//
// MFMA v_mfma_f32_32x32x16_bf16: A lane l holds row l%32, k = 8(l/32) .. +7; B lane l holds
// column l%32, same k; the result's register v in lane l is row 8(v/4) + 4(l/32) + v%4,
// column l%32.

#pragma once

#include "attn_device.h"

namespace attn {

// launches the head_dim 256 dk/dv and dq kernels (attn_bwd_d256.hip)
hipError_t launch_bwd_d256_main(const BwdParams &p, const RopeTable &tab, hipStream_t stream);

namespace {

constexpr int BR = 32;  // rows per block

__device__ __forceinline__ f32x16 bwd_mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Workgroup i runs on XCD i % 8 (round-robin dispatch).  This renumbers the n workgroups so
// that each XCD gets a contiguous run of the logical order, i.e. the blocks of the same K/V
// head group, whose tiles then stay in that XCD's L2.  A bijection on [0, n) for any n.
__device__ __forceinline__ int xcd_order(int i, int n) {
  const int x = i & 7, q = n >> 3, r = n & 7;
  return x * q + min(x, r) + (i >> 3);
}

__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// floor(a / b) for b > 0 and any sign of a
__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

__device__ __forceinline__ bf16x8 ld16(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// 16 bytes at byte voff (per lane) + soff (uniform) of a buffer: the base stays in scalar
// registers and each lane keeps one 32-bit offset, not a 64-bit address per operand stream.
// Constant parts of an offset go into soff, so that no lane holds a register per operand.
__device__ __forceinline__ u32x4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

// Row of result register v in lane half hh.
__device__ __forceinline__ int res_row(int v, int hh) { return 8 * (v >> 2) + 4 * hh + (v & 3); }

// Writes a 32-row block staged in LDS (rows of stride LS elements) in "t" layout: 4*D chunks of
// 16 bytes, chunk (half, j, column) = rows 16 half + swap23(8 j + e), e = 0..7, of that column.
template <int D, int LS>
__device__ __forceinline__ void write_t_layout(const uint16_t *lds, __bf16 *dst, int tid, int nthreads) {
  for (int ch = tid; ch < 4 * D; ch += nthreads) {
    const int col = ch % D;
    const int hj = ch / D;  // 2 half + j
    const int half = hj >> 1, j = hj & 1;
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int r0 = 16 * half + swap23(8 * j + e);
      const int r1 = 16 * half + swap23(8 * j + e + 1);
      w[e / 2] = (uint32_t)lds[r0 * LS + col] | ((uint32_t)lds[r1 * LS + col] << 16);
    }
    *reinterpret_cast<u32x4 *>(dst + (size_t)ch * 8) = w;
  }
}

// Rotation of 8 pairs (x_i, y_i) = (dims 8c + i, D/2 + 8c + i) of one row at position pos.
template <int D>
__device__ __forceinline__ void rotate8(const RopeTable &tab, int c, int pos, const u32x4 &xr, const u32x4 &yr,
                                        float x[8], float y[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t xw = xr[i / 2], yw = yr[i / 2];
    const float xv = (i & 1) ? bf16_hi(xw) : bf16_lo(xw);
    const float yv = (i & 1) ? bf16_hi(yw) : bf16_lo(yw);
    const float t = turn_fraction(pos, tab.rev[8 * c + i]);
    const float sn = __builtin_amdgcn_sinf(t), cs = __builtin_amdgcn_cosf(t);
    x[i] = xv * cs - yv * sn;
    y[i] = yv * cs + xv * sn;
  }
}

__device__ __forceinline__ u32x4 pack8(const float a[8], float s) {
  return u32x4{pack_bf16x2(a[0] * s, a[1] * s), pack_bf16x2(a[2] * s, a[3] * s), pack_bf16x2(a[4] * s, a[5] * s),
               pack_bf16x2(a[6] * s, a[7] * s)};
}

}  // namespace

}  // namespace attn
