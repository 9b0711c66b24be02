// C ABI of the attention forward (declared in include/attn.h): host-side validation,
// kernel selection and launch.  Every argument is checked before the first HIP runtime
// call, so a rejected call enqueues nothing.

#include "attn.h"

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <random>

#include "attn_launch.h"

#define ATTN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kTileKeys = 64;  // key tile of the bf16 kernel; prepared K and V are padded to it

size_t padded_len(int S) { return ((size_t)S + kTileKeys - 1) / kTileKeys * kTileKeys; }

// Prepared tiles of the bf16 forward: rotated keys, then transposed values.
size_t tile_bytes(int B, int S, int Hkv, int d) { return 2 * (size_t)B * Hkv * padded_len(S) * d * 2; }

// After the tiles, the one-launch form's flags (one 8-byte tag per tile half) and a status word.
size_t flag_bytes(int B, int S, int Hkv) {
  const size_t n = (size_t)B * Hkv * (padded_len(S) / kTileKeys) * 2;
  return (n * 8 + 16 + 255) / 256 * 256;
}

// Tags of one-launch calls: a process-wide counter started at a random 64-bit value, so a tag
// equals a value left in a workspace by an earlier call (or by anything else) only by chance,
// with probability 2^-64 per flag; 0 is skipped.
unsigned long long next_call_tag() {
  static std::atomic<unsigned long long> counter{[] {
    std::random_device rd;
    unsigned long long s = ((unsigned long long)rd() << 32) ^ rd();
    s ^= (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    return s;
  }()};
  unsigned long long t = counter.fetch_add(1, std::memory_order_relaxed);
  if (t == 0) t = counter.fetch_add(1, std::memory_order_relaxed);
  return t;
}

// Whether a bf16 forward of this grid takes the one-launch form: every workgroup must be
// resident at once, and each wave group prepares at most kMaxPrepRounds tile halves (measured:
// the one-launch form is as fast or faster up to 8 on the SmolLM MHA shape, B 4, S 1024, 32
// heads of 64, and 1 on the Llama-3-8B and PaLM MQA shapes; a larger count would move more of
// the preparation into the prologue than the separate pass costs).  The environment
// variable ATTN_FWD_PATH = "split" or "fused" overrides the choice (a diagnostic; "fused" is
// still refused when the grid would not be resident).
constexpr int kMaxPrepRounds = 8;

// Bound of the one-launch form's wait for published tiles: each poll is a device-scope read
// plus a ~0.1 us sleep, so the bound is a fraction of a second; the wait normally ends within
// a few microseconds.
constexpr int kMaxPolls = 1 << 18;

template <int D>
bool choose_fused(long long blocks, bool dual, int prep_rounds) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return false;
  static std::atomic<int> per_cu[2] = {{-1}, {-1}};
  int n = per_cu[dual].load(std::memory_order_relaxed);
  if (n < 0) {
    n = attn::fwd_bf16_wgs_per_cu<D>(dual);
    per_cu[dual].store(n, std::memory_order_relaxed);
  }
  if (blocks > (long long)cus * n) return false;
  const char *env = std::getenv("ATTN_FWD_PATH");
  if (env && std::strcmp(env, "split") == 0) return false;
  if (env && std::strcmp(env, "fused") == 0) return true;
  return prep_rounds <= kMaxPrepRounds;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Query heads per 4-wave group: the largest of 4, 2, 1 dividing G.
int heads_per_group(int G) { return G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1); }

int check_shape(int B, int S, int Hq, int Hkv, int d, double rope_theta, int causal, int dtype) {
  if (B < 1 || S < 1 || Hq < 1 || Hkv < 1) return ATTN_EINVAL;
  if (Hq % Hkv != 0) return ATTN_EINVAL;
  if (!std::isfinite(rope_theta) || rope_theta <= 0.0) return ATTN_EINVAL;
  if (causal != 0 && causal != 1) return ATTN_EINVAL;
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_FP32) return ATTN_EUNSUPPORTED;
  if (d != 64 && d != 128 && !(d == 256 && dtype == ATTN_DTYPE_BF16)) return ATTN_EUNSUPPORTED;
  // index arithmetic in the kernels: row/key positions in int, offsets in size_t,
  // workgroup counts below 2^31
  if (S > (1 << 28)) return ATTN_EUNSUPPORTED;
  // the kernels address one (b, head) run of prepared tiles (S padded to 64 keys, d bf16 per
  // key) with 32-bit buffer offsets
  if ((double)padded_len(S) * d * 2 >= 2147483647.0) return ATTN_EUNSUPPORTED;
  if ((double)Hkv * d > (double)(1 << 24)) return ATTN_EUNSUPPORTED;  // 32-bit offsets within a 64-key tile
  const double elems = (double)B * S * Hq * d;
  if (elems > 4.0e15) return ATTN_EUNSUPPORTED;
  const double wgs = (double)B * Hq * ((double)S / 32.0 + 1.0) + (double)B * Hkv * (padded_len(S) / 256.0 + 1.0) * (d / 16);
  if (wgs >= 2147483647.0) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

bool rope_style_ok(int rope_style) { return rope_style == ATTN_ROPE_HALF || rope_style == ATTN_ROPE_INTERLEAVED; }

attn::RopeTable rope_table(int d, double rope_theta, int rope_style) {
  attn::RopeTable t{};
  t.interleaved = rope_style == ATTN_ROPE_INTERLEAVED;
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < d / 2; ++i) t.rev[i] = std::pow(rope_theta, -(2.0 * i) / d) / two_pi;
  return t;
}

float q_scale(int d) { return (float)(1.4426950408889634073599246810019 / std::sqrt((double)d)); }

template <int D>
hipError_t run_bf16(const void *q, const void *k, const void *v, int B, int S, int Hq, int Hkv,
                    const attn::RopeTable &tab, int causal, int q_pos0, int k_pos0, void *out,
                    float *lse, void *ws, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const size_t s_pad = padded_len(S);
  __bf16 *kr = static_cast<__bf16 *>(ws);
  __bf16 *vt = kr + (size_t)B * Hkv * s_pad * D;

  attn::FwdParams p{};
  p.q = static_cast<const __bf16 *>(q);
  p.kr = kr;
  p.vt = vt;
  p.out = static_cast<__bf16 *>(out);
  p.lse = lse;
  p.B = B;
  p.S = S;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.S_pad = (int)s_pad;
  p.hpw = heads_per_group(p.G);
  p.rows_per_blk = 32 * (4 / p.hpw);
  p.n_units = B * Hkv * (p.G / p.hpw);
  p.n_row_blocks = (S + p.rows_per_blk - 1) / p.rows_per_blk;
  p.n_pairs = (p.n_row_blocks + 1) / 2;
  p.q_pos0 = q_pos0;
  p.delta = q_pos0 - k_pos0;
  p.q_scale = q_scale(D);
  // head_dim 64 keeps its LDS small enough for each wave group to run a unit of its own: when
  // the (unit, pair) items outnumber the CUs, pairs of units share a workgroup and the grid runs
  // in one round instead of two
  p.dual = 0;
  if (D == 64 && p.n_units % 2 == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      p.dual = (long long)p.n_units * p.n_pairs > cus ? 1 : 0;
  }

  if constexpr (D != 256) {
    // one launch when the whole grid is resident: the attention kernel prepares the tiles
    p.k = static_cast<const __bf16 *>(k);
    p.v = static_cast<const __bf16 *>(v);
    p.k_pos0 = k_pos0;
    p.prep_workers = (p.G / p.hpw) * p.n_pairs * (p.dual ? 1 : 2);
    const int n_jobs = 2 * (int)(s_pad / kTileKeys);
    p.prep_rounds = (n_jobs + p.prep_workers - 1) / p.prep_workers;
    const long long blocks = (long long)p.n_pairs * (p.dual ? p.n_units / 2 : p.n_units);
    if (choose_fused<D>(blocks, p.dual != 0, p.prep_rounds)) {
      char *fl = reinterpret_cast<char *>(ws) + tile_bytes(B, S, Hkv, D);
      p.flags = reinterpret_cast<unsigned long long *>(fl);
      p.status = reinterpret_cast<unsigned int *>(fl + (size_t)B * Hkv * (s_pad / kTileKeys) * 2 * 8);
      p.tag = next_call_tag();
      p.await_tag = p.tag;
      p.max_polls = kMaxPolls;
      const char *force = std::getenv("ATTN_FWD_FORCE_TIMEOUT");
      if (force && std::strcmp(force, "1") == 0) {
        // diagnostic: every wait looks for a tag no workgroup writes and gives up after a few
        // polls, so the timeout path runs with every kernel exiting normally
        p.await_tag = p.tag ^ 1ull;
        p.max_polls = 4;
      }
      return causal ? attn::launch_attn_bf16<D, true>(p, tab, st, e0, e1)
                    : attn::launch_attn_bf16<D, false>(p, tab, st, e0, e1);
    }
  }

  attn::PrepParams pp;
  pp.k = static_cast<const __bf16 *>(k);
  pp.v = static_cast<const __bf16 *>(v);
  pp.kr = kr;
  pp.vt = vt;
  pp.B = B;
  pp.S = S;
  pp.Hkv = Hkv;
  pp.S_pad = (int)s_pad;
  pp.S_rows = S;
  pp.tile0 = 0;
  pp.n_run = (int)(s_pad / kTileKeys);
  pp.k_pos0 = k_pos0;
  hipError_t err = attn::launch_prep_kv<D>(pp, tab, st);
  if (err != hipSuccess) return err;
  p.flags = nullptr;
  if constexpr (D == 256) {
    return causal ? attn::launch_attn_d256<true>(p, tab, st, e0, e1) : attn::launch_attn_d256<false>(p, tab, st, e0, e1);
  } else {
    return causal ? attn::launch_attn_bf16<D, true>(p, tab, st, e0, e1)
                  : attn::launch_attn_bf16<D, false>(p, tab, st, e0, e1);
  }
}

template <int D>
hipError_t run_f32(const void *q, const void *k, const void *v, int B, int S, int Hq, int Hkv,
                   const attn::RopeTable &tab, int causal, int q_pos0, int k_pos0, void *out,
                   float *lse, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  attn::F32Params p;
  p.q = static_cast<const float *>(q);
  p.k = static_cast<const float *>(k);
  p.v = static_cast<const float *>(v);
  p.out = static_cast<float *>(out);
  p.lse = lse;
  p.B = B;
  p.S = S;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.n_row_blocks = (S + 63) / 64;
  p.q_pos0 = q_pos0;
  p.k_pos0 = k_pos0;
  p.q_scale = q_scale(D);
  return causal ? attn::launch_attn_f32<D, true>(p, tab, st, e0, e1)
                : attn::launch_attn_f32<D, false>(p, tab, st, e0, e1);
}

int fwd_impl(const void *q, const void *k, const void *v, int B, int S, int Hq, int Hkv, int d,
             double rope_theta, int rope_style, int causal, int q_pos0, int k_pos0, int dtype, void *out, float *lse,
             void *workspace, size_t workspace_bytes, void *stream, void *ev_start, void *ev_stop) {
  if (!q || !k || !v || !out || !lse) return ATTN_EINVAL;
  // positions (offset + row) stay below 2^30, so every position difference fits an int
  if (q_pos0 < 0 || k_pos0 < 0 || (long long)q_pos0 + S > (1LL << 30) || (long long)k_pos0 + S > (1LL << 30))
    return ATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(lse, 4))
    return ATTN_EINVAL;
  if (!rope_style_ok(rope_style)) return ATTN_EINVAL;
  const int rc = check_shape(B, S, Hq, Hkv, d, rope_theta, causal, dtype);
  if (rc != ATTN_OK) return rc;
  const size_t need = attn_fwd_workspace_bytes(B, S, Hkv, d, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16))) return ATTN_EWORKSPACE;

  const attn::RopeTable tab = rope_table(d, rope_theta, rope_style);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = static_cast<hipEvent_t>(ev_start), e1 = static_cast<hipEvent_t>(ev_stop);
  hipError_t err;
  if (dtype == ATTN_DTYPE_BF16)
    err = d == 64    ? run_bf16<64>(q, k, v, B, S, Hq, Hkv, tab, causal, q_pos0, k_pos0, out, lse, workspace, st, e0, e1)
          : d == 128 ? run_bf16<128>(q, k, v, B, S, Hq, Hkv, tab, causal, q_pos0, k_pos0, out, lse, workspace, st, e0, e1)
                     : run_bf16<256>(q, k, v, B, S, Hq, Hkv, tab, causal, q_pos0, k_pos0, out, lse, workspace, st, e0, e1);
  else
    err = d == 64 ? run_f32<64>(q, k, v, B, S, Hq, Hkv, tab, causal, q_pos0, k_pos0, out, lse, st, e0, e1)
                  : run_f32<128>(q, k, v, B, S, Hq, Hkv, tab, causal, q_pos0, k_pos0, out, lse, st, e0, e1);
  return err == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

}  // namespace

ATTN_EXPORT int attn_abi_version(void) { return ATTN_ABI_VERSION; }

ATTN_EXPORT const char *attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "success";
    case ATTN_EINVAL: return "invalid argument (null/misaligned pointer, non-positive size, Hq not a multiple of Hkv, bad rope_theta, rope_style or causal flag)";
    case ATTN_EUNSUPPORTED: return "unsupported configuration (head_dim must be 64 or 128, or 256 for the bf16 calls but not float32; dtype bf16 or fp32; sizes within limits)";
    case ATTN_EHIP: return "HIP runtime error while recording an event or launching a kernel";
    case ATTN_EWORKSPACE: return "workspace missing, misaligned or smaller than attn_fwd_workspace_bytes()";
    case ATTN_ESCRATCH: return "attn_fwd_noalloc: the call needs more workspace than the library's fixed scratch (ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

ATTN_EXPORT size_t attn_fwd_workspace_bytes(int B, int S, int Hkv, int head_dim, int dtype) {
  if (dtype != ATTN_DTYPE_BF16) return 0;
  if (B < 1 || S < 1 || Hkv < 1 || (head_dim != 64 && head_dim != 128 && head_dim != 256) || S > (1 << 28)) return 0;
  // rotated K and transposed V, then the one-launch form's flags
  return tile_bytes(B, S, Hkv, head_dim) + (head_dim != 256 ? flag_bytes(B, S, Hkv) : 0);
}

ATTN_EXPORT int attn_fwd(const void *q, const void *k, const void *v, int B, int S, int Hq, int Hkv,
                         int head_dim, double rope_theta, int rope_style, int causal, int dtype, void *out,
                         float *lse, void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_impl(q, k, v, B, S, Hq, Hkv, head_dim, rope_theta, rope_style, causal, 0, 0, dtype, out, lse, workspace,
                  workspace_bytes, stream, nullptr, nullptr);
}

ATTN_EXPORT int attn_fwd_shard(const void *q, const void *k, const void *v, int B, int S, int Hq, int Hkv,
                               int head_dim, double rope_theta, int rope_style, int causal, int q_pos0,
                               int k_pos0, int dtype, void *out, float *lse, void *workspace,
                               size_t workspace_bytes, void *stream) {
  return fwd_impl(q, k, v, B, S, Hq, Hkv, head_dim, rope_theta, rope_style, causal, q_pos0, k_pos0, dtype, out, lse,
                  workspace, workspace_bytes, stream, nullptr, nullptr);
}

ATTN_EXPORT int attn_merge(const void *o1, const float *lse1, const void *o2, const float *lse2, int B, int S,
                           int H, int head_dim, int dtype, void *out, float *lse, void *stream) {
  if (!o1 || !lse1 || !o2 || !lse2 || !out || !lse) return ATTN_EINVAL;
  if (!aligned(o1, 16) || !aligned(o2, 16) || !aligned(out, 16) || !aligned(lse1, 4) || !aligned(lse2, 4) ||
      !aligned(lse, 4))
    return ATTN_EINVAL;
  if (B < 1 || S < 1 || H < 1) return ATTN_EINVAL;
  if (dtype != ATTN_DTYPE_BF16 && dtype != ATTN_DTYPE_FP32) return ATTN_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256) return ATTN_EUNSUPPORTED;
  const double rows = (double)B * S * H;
  if (rows * (head_dim / 4) >= 2147483647.0 * 256.0 || rows * head_dim > 4.0e15) return ATTN_EUNSUPPORTED;
  attn::MergeParams p;
  p.o1 = o1;
  p.o2 = o2;
  p.lse1 = lse1;
  p.lse2 = lse2;
  p.out = out;
  p.lse = lse;
  p.rows = (long long)B * S * H;
  p.S = S;
  p.H = H;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (dtype == ATTN_DTYPE_BF16)
    err = head_dim == 64    ? attn::launch_merge<__bf16, 64>(p, st)
          : head_dim == 128 ? attn::launch_merge<__bf16, 128>(p, st)
                            : attn::launch_merge<__bf16, 256>(p, st);
  else
    err = head_dim == 64    ? attn::launch_merge<float, 64>(p, st)
          : head_dim == 128 ? attn::launch_merge<float, 128>(p, st)
                            : attn::launch_merge<float, 256>(p, st);
  return err == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

namespace {

// Workspace of attn_fwd_noalloc: one array per GPU in the library's device memory.  Host code
// uses only the device address that hipGetSymbolAddress returns for the current device (the
// array's own name is a host-side stand-in, not a device address).
__device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of the current device's scratch, looked up once per device (concurrent first
// calls may both look it up; they store the same address).  nullptr on failure.
void *scratch_for(int dev) {
  static std::atomic<void *> addr[kMaxDevices];
  void *ptr = addr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    addr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

ATTN_EXPORT int attn_fwd_noalloc(const void *q, const void *k, const void *v, int B, int S, int Hq, int Hkv,
                                 int head_dim, double rope_theta, int rope_style, int causal, int dtype, void *out,
                                 float *lse, void *stream) {
  // the arguments attn_fwd checks first, so that a rejected call touches no device state
  if (!q || !k || !v || !out || !lse) return ATTN_EINVAL;
  const int rc = check_shape(B, S, Hq, Hkv, head_dim, rope_theta, causal, dtype);
  if (rc != ATTN_OK) return rc;
  const size_t need = attn_fwd_workspace_bytes(B, S, Hkv, head_dim, dtype);
  if (need > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ESCRATCH;
  void *ws = nullptr;
  if (need > 0) {
    int dev = -1, sdev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_EHIP;
    if (stream != nullptr && (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess || sdev != dev))
      return ATTN_EINVAL;
    ws = scratch_for(dev);
    if (ws == nullptr) return ATTN_EHIP;
  }
  return fwd_impl(q, k, v, B, S, Hq, Hkv, head_dim, rope_theta, rope_style, causal, 0, 0, dtype, out, lse, ws,
                  need, stream, nullptr, nullptr);
}

ATTN_EXPORT int attn_fwd_timed(const void *q, const void *k, const void *v, int B, int S, int Hq, int Hkv,
                               int head_dim, double rope_theta, int rope_style, int causal, int dtype,
                               void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream,
                               void *ev_start, void *ev_stop) {
  return fwd_impl(q, k, v, B, S, Hq, Hkv, head_dim, rope_theta, rope_style, causal, 0, 0, dtype, out, lse, workspace,
                  workspace_bytes, stream, ev_start, ev_stop);
}

ATTN_EXPORT void *attn_event_create(void) {
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

namespace {

// Decode splits: about kDecodeWaves waves over (b, K/V head, head block, key range), i.e. four
// per CU, one per SIMD, at least kDecodeMinHalves 32-key half tiles per key range so that each
// wave's loads fill its pipeline, and at most kDecodeMaxSplits ranges per (b, K/V head, head
// block), past which the join's rows and the ranges' start-up cost more than the extra waves
// gain (measured: a 32K cache at batch 1 and Llama-3-8B heads decodes faster with 64 ranges of
// 512 keys than with 128 of 256).  A workgroup is one wave, two at head_dim 256.
constexpr int kDecodeWaves = 1024;
constexpr int kDecodeMinHalves = 4;
constexpr int kDecodeMaxSplits = 64;

int decode_hblk(int G) { return (G + 31) / 32; }

int decode_max_splits(int B, int Hkv, int G, int d) {
  const long long units = (long long)B * Hkv * decode_hblk(G);
  const long long wgs = kDecodeWaves / (d == 256 ? 2 : 1);
  return (int)std::max<long long>(1, std::min<long long>(kDecodeMaxSplits, (wgs + units - 1) / units));
}

int check_decode_shape(int B, int S_cap, int Hq, int Hkv, int d) {
  if (B < 1 || S_cap < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_EINVAL;
  if (d != 64 && d != 128 && d != 256) return ATTN_EUNSUPPORTED;
  if (S_cap > (1 << 28) || (double)Hkv * d > (double)(1 << 24)) return ATTN_EUNSUPPORTED;
  // one (b, g) tile run of the cache is addressed with 32-bit offsets
  if ((double)padded_len(S_cap) * d * 2 >= 2147483647.0) return ATTN_EUNSUPPORTED;
  if ((double)B * Hq > (double)(1 << 24)) return ATTN_EUNSUPPORTED;  // one join workgroup per (b, head)
  return ATTN_OK;
}

}  // namespace

ATTN_EXPORT int attn_kv_prepare(const void *k, const void *v, int B, int S_cap, int Hkv, int head_dim,
                                double rope_theta, int rope_style, int key0, int key1, void *cache,
                                size_t cache_bytes, void *stream) {
  if (!k || !v || !cache) return ATTN_EINVAL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(cache, 16)) return ATTN_EINVAL;
  const int rc = check_decode_shape(B, S_cap, Hkv, Hkv, head_dim);
  if (rc != ATTN_OK) return rc;
  if (!std::isfinite(rope_theta) || rope_theta <= 0.0 || !rope_style_ok(rope_style)) return ATTN_EINVAL;
  if (key0 < 0 || key1 <= key0 || key1 > S_cap) return ATTN_EINVAL;
  if (cache_bytes < attn_fwd_workspace_bytes(B, S_cap, Hkv, head_dim, ATTN_DTYPE_BF16)) return ATTN_EWORKSPACE;
  const size_t s_pad = padded_len(S_cap);
  attn::PrepParams pp;
  pp.k = static_cast<const __bf16 *>(k);
  pp.v = static_cast<const __bf16 *>(v);
  pp.kr = static_cast<__bf16 *>(cache);
  pp.vt = pp.kr + (size_t)B * Hkv * s_pad * head_dim;
  pp.B = B;
  pp.S = key1;
  pp.Hkv = Hkv;
  pp.S_pad = (int)s_pad;
  pp.S_rows = S_cap;
  pp.tile0 = key0 / kTileKeys;
  pp.n_run = (key1 + kTileKeys - 1) / kTileKeys - pp.tile0;
  pp.k_pos0 = 0;
  const attn::RopeTable tab = rope_table(head_dim, rope_theta, rope_style);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t err = head_dim == 64    ? attn::launch_prep_kv<64>(pp, tab, st)
                         : head_dim == 128 ? attn::launch_prep_kv<128>(pp, tab, st)
                                           : attn::launch_prep_kv<256>(pp, tab, st);
  return err == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

ATTN_EXPORT size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int head_dim) {
  if (check_decode_shape(B, 1, Hq, Hkv, head_dim) != ATTN_OK) return 0;
  const size_t rows = (size_t)B * Hq * decode_max_splits(B, Hkv, Hq / Hkv, head_dim);
  return rows * ((size_t)head_dim + 2) * sizeof(float);
}

namespace {

// attn_decode and attn_decode_ragged: q_pos is the batch's position, or with q_pos_rows the
// largest position a row may have.
int decode_impl(const void *q, const void *cache, size_t cache_bytes, int B, int S_cap, int Hq, int Hkv,
                int head_dim, double rope_theta, int rope_style, int q_pos, const int *q_pos_rows, void *out,
                float *lse, void *workspace, size_t workspace_bytes, void *stream) {
  if (!q || !cache || !out || !lse) return ATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(out, 16) || !aligned(lse, 4)) return ATTN_EINVAL;
  const int rc = check_decode_shape(B, S_cap, Hq, Hkv, head_dim);
  if (rc != ATTN_OK) return rc;
  if (!std::isfinite(rope_theta) || rope_theta <= 0.0 || !rope_style_ok(rope_style)) return ATTN_EINVAL;
  if (q_pos < 0 || q_pos >= S_cap) return ATTN_EINVAL;
  // the kernels address the V^T half at B * Hkv * S_cap (padded) * head_dim past the start: the
  // cache must hold the whole layout for these sizes
  if (cache_bytes < attn_fwd_workspace_bytes(B, S_cap, Hkv, head_dim, ATTN_DTYPE_BF16)) return ATTN_EWORKSPACE;
  const size_t need = attn_decode_workspace_bytes(B, Hq, Hkv, head_dim);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return ATTN_EWORKSPACE;
  const size_t s_pad = padded_len(S_cap);
  const int G = Hq / Hkv;
  attn::DecodeParams p;
  p.q = static_cast<const __bf16 *>(q);
  p.kr = static_cast<const __bf16 *>(cache);
  p.vt = p.kr + (size_t)B * Hkv * s_pad * head_dim;
  p.out = static_cast<__bf16 *>(out);
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = G;
  p.S_pad = (int)s_pad;
  p.q_pos = q_pos;
  p.q_pos_rows = q_pos_rows;
  p.n_hblk = decode_hblk(G);
  const int halves = (q_pos + 1 + 31) / 32;
  const int max_split = std::max(1, std::min(decode_max_splits(B, Hkv, G, head_dim), halves / kDecodeMinHalves));
  p.halves_per_split = (halves + max_split - 1) / max_split;
  p.n_split = (halves + p.halves_per_split - 1) / p.halves_per_split;
  const size_t rows = (size_t)B * Hq * p.n_split;
  p.po = static_cast<float *>(workspace);
  p.pm = p.po + rows * head_dim;
  p.pl = p.pm + rows;
  p.q_scale = q_scale(head_dim);
  const attn::RopeTable tab = rope_table(head_dim, rope_theta, rope_style);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t err = head_dim == 64    ? attn::launch_decode<64>(p, tab, st)
                         : head_dim == 128 ? attn::launch_decode<128>(p, tab, st)
                                           : attn::launch_decode<256>(p, tab, st);
  return err == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

}  // namespace

ATTN_EXPORT int attn_decode(const void *q, const void *cache, size_t cache_bytes, int B, int S_cap, int Hq,
                            int Hkv, int head_dim, double rope_theta, int rope_style, int q_pos, void *out,
                            float *lse, void *workspace, size_t workspace_bytes, void *stream) {
  return decode_impl(q, cache, cache_bytes, B, S_cap, Hq, Hkv, head_dim, rope_theta, rope_style, q_pos, nullptr, out,
                     lse, workspace, workspace_bytes, stream);
}

ATTN_EXPORT int attn_decode_ragged(const void *q, const void *cache, size_t cache_bytes, int B, int S_cap, int Hq,
                                   int Hkv, int head_dim, double rope_theta, int rope_style, const int *q_pos,
                                   int max_pos, void *out, float *lse, void *workspace, size_t workspace_bytes,
                                   void *stream) {
  if (!q_pos || !aligned(q_pos, 4)) return ATTN_EINVAL;
  return decode_impl(q, cache, cache_bytes, B, S_cap, Hq, Hkv, head_dim, rope_theta, rope_style, max_pos, q_pos, out,
                     lse, workspace, workspace_bytes, stream);
}

namespace {

constexpr int kBwdRows = 32;  // query and key block of the backward kernels

size_t bwd_blocks(int S) { return ((size_t)S + kBwdRows - 1) / kBwdRows; }

// Head splits of the dk/dv kernels at head_dim 256: a (b, g, key-block pair) workgroup takes its
// group's query heads W = min(G, 4) at a time; when there are few such workgroups and several passes of
// heads (PaLM-540B: 32 workgroups, 12 passes), the passes are spread over HS workgroups that
// leave fp32 partial sums for a reduction kernel.  Aimed at kBwdTargetGroups workgroups (two
// per CU of a 256-CU GPU); a function of the shapes only, so the workspace size is too.
constexpr long long kBwdTargetGroups = 512;

int bwd_head_splits_pairs(int B, int Hkv, int G, size_t nb) {
  const int W = std::min(G, 4);
  const long long passes = (G + W - 1) / W;
  const long long groups = (long long)B * Hkv * (long long)((nb + 1) / 2);
  const long long want = (kBwdTargetGroups + groups - 1) / groups;
  return (int)std::max(1LL, std::min(passes, want));
}

// head_dim 64 and 128: the dk/dv kernels share each query block between four consecutive key
// blocks (one wave each) and run a head split's query heads one after another; the splits are
// aimed at kBwdTargetWaves waves (two per SIMD of a 256-CU GPU), at most one per head.  A
// function of the shapes only, so the workspace size is too.
constexpr long long kBwdTargetWaves = 2048;

int bwd_head_splits(int B, int Hkv, int G, size_t nb, int head_dim) {
  if (head_dim == 256) return bwd_head_splits_pairs(B, Hkv, G, nb);
  const long long waves = (long long)B * Hkv * (long long)((nb + 3) / 4) * 4;
  const long long want = (kBwdTargetWaves + waves - 1) / waves;
  return (int)std::max(1LL, std::min((long long)G, want));
}

}  // namespace

ATTN_EXPORT size_t attn_bwd_workspace_bytes(int B, int S, int Hq, int Hkv, int head_dim) {
  if (check_shape(B, S, Hq, Hkv, head_dim, 1.0, 1, ATTN_DTYPE_BF16) != ATTN_OK) return 0;
  const size_t nb = bwd_blocks(S);
  const size_t tile = (size_t)kBwdRows * head_dim * 2;
  const int hs = bwd_head_splits(B, Hkv, Hq / Hkv, nb, head_dim);
  const size_t part = hs > 1 ? 2 * (size_t)hs * B * Hkv * nb * kBwdRows * head_dim * 4 : 0;
  return 3 * (size_t)B * Hkv * nb * tile + 4 * (size_t)B * Hq * nb * tile + 2 * (size_t)B * Hq * nb * kBwdRows * 4 + part;
}

ATTN_EXPORT int attn_bwd_shard(const void *q, const void *k, const void *v, const void *out, const float *lse,
                               const void *dout, int B, int S, int Hq, int Hkv, int head_dim, double rope_theta,
                               int rope_style, int causal, int q_pos0, int k_pos0, void *dq, void *dk, void *dv,
                               void *workspace, size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !out || !lse || !dout || !dq || !dk || !dv) return ATTN_EINVAL;
  if (q_pos0 < 0 || k_pos0 < 0 || (long long)q_pos0 + S > (1LL << 30) || (long long)k_pos0 + S > (1LL << 30))
    return ATTN_EINVAL;
  for (const void *ptr : {q, k, v, out, dout, (const void *)dq, (const void *)dk, (const void *)dv})
    if (!aligned(ptr, 16)) return ATTN_EINVAL;
  if (!aligned(lse, 4) || !rope_style_ok(rope_style)) return ATTN_EINVAL;
  const int rc = check_shape(B, S, Hq, Hkv, head_dim, rope_theta, causal, ATTN_DTYPE_BF16);
  if (rc != ATTN_OK) return rc;
  const size_t nb = bwd_blocks(S);
  if ((double)B * Hq * nb >= 2147483647.0) return ATTN_EUNSUPPORTED;
  const size_t need = attn_bwd_workspace_bytes(B, S, Hq, Hkv, head_dim);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return ATTN_EWORKSPACE;
  const int G = Hq / Hkv;
  const size_t tile = (size_t)kBwdRows * head_dim;  // elements
  attn::BwdParams p;
  p.q = static_cast<const __bf16 *>(q);
  p.k = static_cast<const __bf16 *>(k);
  p.v = static_cast<const __bf16 *>(v);
  p.out = static_cast<const __bf16 *>(out);
  p.dout = static_cast<const __bf16 *>(dout);
  p.lse = lse;
  p.dq = static_cast<__bf16 *>(dq);
  p.dk = static_cast<__bf16 *>(dk);
  p.dv = static_cast<__bf16 *>(dv);
  const size_t kt_n = (size_t)B * Hkv * nb * tile, qt_n = (size_t)B * Hq * nb * tile;
  p.kc = static_cast<__bf16 *>(workspace);
  p.kt = p.kc + kt_n;
  p.vc = p.kt + kt_n;
  p.qc = p.vc + kt_n;
  p.qt = p.qc + qt_n;
  p.dc = p.qt + qt_n;
  p.dt = p.dc + qt_n;
  p.l2 = reinterpret_cast<float *>(p.dt + qt_n);
  p.dd = p.l2 + (size_t)B * Hq * nb * kBwdRows;
  p.part = p.dd + (size_t)B * Hq * nb * kBwdRows;
  p.HS = bwd_head_splits(B, Hkv, G, nb, head_dim);
  p.B = B;
  p.S = S;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = G;
  p.NB = (int)nb;
  p.n_pairs = (int)((nb + 1) / 2);
  p.W = std::min(G, 4);
  p.causal = causal;
  p.q_pos0 = q_pos0;
  p.k_pos0 = k_pos0;
  p.scale_log2 = q_scale(head_dim);
  p.inv_sqrt_d = (float)(1.0 / std::sqrt((double)head_dim));
  const attn::RopeTable tab = rope_table(head_dim, rope_theta, rope_style);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t err = head_dim == 64    ? attn::launch_bwd<64>(p, tab, st)
                         : head_dim == 128 ? attn::launch_bwd<128>(p, tab, st)
                                           : attn::launch_bwd<256>(p, tab, st);
  return err == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

ATTN_EXPORT int attn_bwd(const void *q, const void *k, const void *v, const void *out, const float *lse,
                         const void *dout, int B, int S, int Hq, int Hkv, int head_dim, double rope_theta,
                         int rope_style, int causal, void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes,
                         void *stream) {
  return attn_bwd_shard(q, k, v, out, lse, dout, B, S, Hq, Hkv, head_dim, rope_theta, rope_style, causal, 0, 0, dq, dk,
                        dv, workspace, workspace_bytes, stream);
}

ATTN_EXPORT int attn_event_destroy(void *ev) {
  if (!ev) return ATTN_EINVAL;
  return hipEventDestroy(static_cast<hipEvent_t>(ev)) == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

ATTN_EXPORT int attn_event_elapsed_ms(void *start, void *stop, float *ms) {
  if (!start || !stop || !ms) return ATTN_EINVAL;
  if (hipEventSynchronize(static_cast<hipEvent_t>(stop)) != hipSuccess) return ATTN_EHIP;
  return hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(stop)) == hipSuccess
             ? ATTN_OK
             : ATTN_EHIP;
}
