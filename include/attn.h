/*
 * attn.h -- C ABI of a fused causal self-attention forward for AMD MI355X (gfx950).
 *
 * One call computes, for every batch row b, query head h and query position i:
 *
 *   q' = RoPE(q[b,i,h,:], i),  k'_j = RoPE(k[b,j,g,:], j),  g = h / (Hq / Hkv)
 *   s_j = q' . k'_j / sqrt(d)           for the visible keys j (j <= i when causal)
 *   out[b,i,h,:] = sum_j softmax(s)_j * v[b,j,g,:]
 *   lse[b,h,i]   = ln sum_j exp(s_j)    (natural log, float32)
 *
 * Definitions followed:
 *   - rotary embedding, half-split form: x*cos + rotate_half(x)*sin with
 *     rotate_half(x) = cat(-x2, x1) over the two halves of head_dim
 *     (Picotron page "Llama architecture and Flash Attention integration", section 1),
 *     frequencies rope_theta^(-2i/d), i < d/2, angle = position * frequency, applied to q
 *     and k only (PaLM-in-ColossalAI page, section 2.3 RotaryEmbedding); or, with
 *     rope_style = ATTN_ROPE_INTERLEAVED, the adjacent-pair form in which dims (2i, 2i+1)
 *     turn together by frequency i, the rotation read as multiplication by complex numbers
 *     (llama3-from-scratch page, rotary position embedding);
 *   - scores scaled by 1/sqrt(head_dim), causal mask on keys later than the query, row
 *     softmax (llama3-from-scratch page: "attention score matrix", "causal mask",
 *     "softmax"); the row maximum is subtracted before exponentiating (PaLM page, 2.5);
 *   - grouped K/V heads: contiguous groups of Hq/Hkv query heads share one K/V head
 *     (llama3 page, "key-value sharing": 32 query heads over 8 K/V heads); Hkv = 1 is
 *     multi-query attention (PaLM page, section 2.5);
 *   - the (B, S, H, D) tensor layout that flash_attn_func receives (Picotron page,
 *     section 2); lse per (head, row) so sequence shards can be merged ring-attention
 *     style (Picotron page, "context parallelism and ring attention").
 *
 * Threading and ownership: every buffer is allocated and owned by the caller; the library
 * allocates no device memory.  Its only mutable global state is a call counter (atomic) that
 * tags the tiles of one-launch forward calls and a per-head_dim cache of the kernel's
 * occupancy, so concurrent calls on different streams are safe as long as their output and
 * workspace buffers do not overlap.
 * Calls are asynchronous: they enqueue work on `stream` and return without synchronising.
 * Every argument is validated on the host before any HIP runtime call; on an error code
 * nothing has been enqueued.  No C++ exception crosses this interface.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 6

/* Element types of q, k, v and out. */
#define ATTN_DTYPE_BF16 0 /* bfloat16 inputs/outputs; bf16 MFMA with float32 accumulation */
#define ATTN_DTYPE_FP32 1 /* float32 inputs/outputs; float32 arithmetic throughout */

/* Rotary pairing (rope_style arguments). */
#define ATTN_ROPE_HALF 0        /* dims (i, i + d/2) form a rotated pair (rotate_half form) */
#define ATTN_ROPE_INTERLEAVED 1 /* dims (2i, 2i + 1) form a rotated pair (complex form) */

/* Return codes. */
#define ATTN_OK 0
#define ATTN_EINVAL (-1)       /* null or misaligned pointer, B/S/Hq/Hkv < 1, Hq % Hkv != 0,
                                  rope_theta not finite or <= 0, rope_style or causal not
                                  0/1 */
#define ATTN_EUNSUPPORTED (-2) /* head_dim not supported by the call (see each call), unknown
                                  dtype, sizes too large (among them S above 2^28, or S rounded
                                  up to 64 times head_dim times 2 bytes at or above 2^31: one
                                  head's run of prepared tiles must fit 32-bit offsets) */
#define ATTN_EHIP (-3)         /* the HIP runtime rejected an event record or kernel launch */
#define ATTN_EWORKSPACE (-4)   /* workspace pointer null while needed, or workspace too small */
#define ATTN_ESCRATCH (-5)     /* attn_fwd_noalloc: the call needs more than the library's
                                  fixed scratch (ATTN_NOALLOC_SCRATCH_BYTES) */

/* Version of this interface (ATTN_ABI_VERSION). */
int attn_abi_version(void);

/* Static, human-readable text for a return code; never NULL. */
const char *attn_strerror(int code);

/*
 * Bytes of device workspace attn_fwd needs for these sizes (0 when none is needed).
 * For bf16 it holds two equal halves of B * Hkv * (S rounded up to 64) * d bf16 elements: the
 * rotated keys, then the values transposed per 64-key tile (a private layout, rewritten on
 * every call).  For head_dim 64 and 128 a flag area follows: one 8-byte tag per half of each
 * 64-key tile, then a 4-byte status word, padded to a multiple of 256 bytes.
 * Returns 0 as well for arguments attn_fwd would reject.
 *
 * How the bf16 forward runs (head_dim 64 and 128).  When every workgroup of the attention
 * kernel fits on the GPU at once, one kernel does everything: each workgroup first rotates the
 * keys (or transposes the values) of a few tiles, writes them through to device scope, tags
 * their flags with a value unique to the call, and then waits until the tiles it reads carry
 * that tag.  Otherwise a separate preparation kernel runs first.  Both give bit-identical
 * results.  The wait is bounded (a fraction of a second); a workgroup whose wait runs out
 * writes NaN to its rows of out and lse and sets the status word to 1 (the library never
 * clears it; a caller who wants to check it zeroes it before the call).  Nothing needs
 * zeroing otherwise: tags left by earlier calls, or any other bytes, are never mistaken for
 * the current call's.  Environment variables, for diagnostics: ATTN_FWD_PATH = "split" forces
 * the separate preparation kernel, "fused" the single kernel wherever the grid fits;
 * ATTN_FWD_FORCE_TIMEOUT = "1" makes every wait of the single kernel run out after a few polls.
 */
size_t attn_fwd_workspace_bytes(int B, int S, int Hkv, int head_dim, int dtype);

/*
 * Fused RoPE + causal (or full) attention forward with grouped K/V heads.
 *
 *   q          device, (B, S, Hq, head_dim) contiguous, element type `dtype`, 16-byte aligned
 *   k, v       device, (B, S, Hkv, head_dim) contiguous, same type, 16-byte aligned
 *   B, S       batch rows and sequence length (>= 1); positions are 0 .. S-1 in every row
 *   Hq, Hkv    query heads and K/V heads; Hq must be a multiple of Hkv
 *   head_dim   64 or 128; also 256 for bf16 (the PaLM page's 540B head size, section 3),
 *              which runs a kernel of its own (split into two rotation halves in every case)
 *   rope_theta rotary base (> 0, finite); frequencies rope_theta^(-2i/head_dim)
 *   rope_style ATTN_ROPE_HALF or ATTN_ROPE_INTERLEAVED: which dims form a rotated pair
 *   causal     1: key j is visible to query i iff j <= i;  0: every key is visible
 *   dtype      ATTN_DTYPE_BF16 or ATTN_DTYPE_FP32
 *   out        device, (B, S, Hq, head_dim) contiguous, type `dtype`, 16-byte aligned;
 *              fully overwritten; must not overlap the inputs
 *   lse        device, (B, Hq, S) float32; fully overwritten
 *   workspace  device scratch of at least attn_fwd_workspace_bytes(...) bytes, 16-byte
 *              aligned (may be NULL when that size is 0); its contents on entry are
 *              ignored and on return are unspecified
 *   stream     hipStream_t to enqueue on; NULL means the default stream
 *
 * Returns ATTN_OK or one of the error codes above.
 */
int attn_fwd(const void *q, const void *k, const void *v, int B, int S, int Hq, int Hkv,
             int head_dim, double rope_theta, int rope_style, int causal, int dtype, void *out,
             float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Same as attn_fwd, and additionally has the runtime record `ev_start` and `ev_stop` with the
 * attention kernel's own dispatch (hipExtLaunchKernel), so the interval between them is that
 * kernel's execution alone; the key/value preparation pass, when there is one, runs before
 * it.  Either event may be NULL.  Events come from attn_event_create.  For benchmarking.
 */
int attn_fwd_timed(const void *q, const void *k, const void *v, int B, int S, int Hq, int Hkv,
                   int head_dim, double rope_theta, int rope_style, int causal, int dtype,
                   void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream,
                   void *ev_start, void *ev_stop);

/*
 * attn_fwd for callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops that must not call hipMalloc, harnesses that forbid it): the same computation,
 * arguments and results, but without a workspace argument.  The workspace is a fixed array of
 * ATTN_NOALLOC_SCRATCH_BYTES in the library's own device memory, one per GPU, held until the
 * process ends; the call allocates nothing (its address is looked up once per device, on the
 * first call there).  A call whose attn_fwd_workspace_bytes(...) exceeds that size returns
 * ATTN_ESCRATCH before any HIP call.  Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (different streams, or different host threads without
 * ordering) race on it and give undefined results; calls ordered on one stream are safe.  The
 * array keeps the last call's contents, and nothing in it needs clearing between calls.
 * The stream must belong to the current device (else ATTN_EINVAL).
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int attn_fwd_noalloc(const void *q, const void *k, const void *v, int B, int S, int Hq, int Hkv,
                     int head_dim, double rope_theta, int rope_style, int causal, int dtype,
                     void *out, float *lse, void *stream);

/*
 * One shard of a longer sequence: attn_fwd for queries at positions q_pos0 .. q_pos0+S-1
 * against keys and values at positions k_pos0 .. k_pos0+S-1 (same S, e.g. one step of ring
 * attention, where each rank attends its query block to the K/V blocks passed around the
 * ring: Picotron page, "context parallelism and ring attention").  The positions rotate q and
 * k, and with causal = 1 key j is visible to query i iff k_pos0 + j <= q_pos0 + i, so an
 * earlier key shard is seen in full, the diagonal one causally, and a later one not at all.
 * A query with no visible key gets out = 0 and lse = -inf, which attn_merge treats as an
 * empty part.  attn_fwd is this call with q_pos0 = k_pos0 = 0.
 *
 *   q_pos0, k_pos0  >= 0, with q_pos0 + S and k_pos0 + S at most 2^30 (else ATTN_EINVAL)
 *   other arguments as for attn_fwd (same workspace size)
 */
int attn_fwd_shard(const void *q, const void *k, const void *v, int B, int S, int Hq, int Hkv,
                   int head_dim, double rope_theta, int rope_style, int causal, int q_pos0,
                   int k_pos0, int dtype, void *out, float *lse, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * Join two partial results for the same queries over disjoint key sets (the merge step of
 * ring attention, Picotron page, context parallelism):
 *   lse = ln(exp(lse1) + exp(lse2)),   out = exp(lse1 - lse) * o1 + exp(lse2 - lse) * o2,
 * with lse the natural-log softmax denominators attn_fwd / attn_fwd_shard return.  A part
 * with lse = -inf contributes nothing; a row empty in both stays out = 0, lse = -inf.
 *
 *   o1, o2, out   device, (B, S, H, head_dim) contiguous, type `dtype`, 16-byte aligned
 *   lse1, lse2, lse  device, (B, H, S) float32, 4-byte aligned
 *   out may be o1 or o2 and lse may be lse1 or lse2 (in-place accumulation); other overlaps
 *   are not allowed.  Computed in float32 and rounded to nearest even into `dtype`.
 * Returns ATTN_OK, ATTN_EINVAL (null or misaligned pointer, B/S/H < 1) or ATTN_EUNSUPPORTED
 * (head_dim not 64, 128 or 256, unknown dtype, sizes too large), ATTN_EHIP on a launch error.
 */
int attn_merge(const void *o1, const float *lse1, const void *o2, const float *lse2, int B, int S,
               int H, int head_dim, int dtype, void *out, float *lse, void *stream);

/*
 * Decode step (the generation loop of the PaLM-in-ColossalAI page, section 2.7, appends one
 * token at a time; section 2.5 notes that sharing one K/V head makes that step cheaper).
 * A key/value cache of capacity S_cap keeps rotated keys and transposed values in the
 * tile layout attn_fwd prepares internally, so each new token re-prepares only its own
 * 64-key tile and attn_decode reads every cached key and value once.  bf16 only; head_dim 64,
 * 128 or 256.
 *
 * attn_kv_prepare: rotate keys [key0, key1) of k at their own positions and store them, with
 * the matching values, into `cache`.  Whole 64-key tiles are rewritten: the tile holding key0
 * is re-read from row 64*floor(key0/64), and keys key1 .. (end of its tile) are stored as
 * zeros, so k and v must hold valid rows [64*floor(key0/64), key1).
 *   k, v     device, (B, S_cap, Hkv, head_dim) bfloat16 contiguous, 16-byte aligned
 *   cache    device, at least attn_fwd_workspace_bytes(B, S_cap, Hkv, head_dim,
 *            ATTN_DTYPE_BF16) bytes, 16-byte aligned, owned by the caller; layout private
 *   rope_style ATTN_ROPE_HALF or ATTN_ROPE_INTERLEAVED, as for attn_fwd
 *   0 <= key0 < key1 <= S_cap
 * Returns ATTN_OK, ATTN_EINVAL (null or misaligned pointer, bad sizes or key range, theta not
 * finite and > 0, bad rope_style), ATTN_EUNSUPPORTED (head_dim not 64, 128 or 256, sizes too large),
 * ATTN_EWORKSPACE (cache too small) or ATTN_EHIP (launch error).
 */
int attn_kv_prepare(const void *k, const void *v, int B, int S_cap, int Hkv, int head_dim,
                    double rope_theta, int rope_style, int key0, int key1, void *cache,
                    size_t cache_bytes, void *stream);

/* Workspace bytes attn_decode needs for these sizes (partial results of its key splits),
 * independent of S_cap and q_pos; 0 for unsupported sizes. */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int head_dim);

/*
 * Decode attention: for every batch row b and query head h, the query q[b, h] at position
 * q_pos (rotated there) attends to cached keys 0 .. q_pos of K/V head h / (Hq/Hkv):
 * the row q_pos of the causal attention attn_fwd computes, with the same scale, rotation and
 * lse.  Keys 0 .. q_pos of `cache` must have been prepared by attn_kv_prepare with the same
 * rope_theta and rope_style.  The key range is split over workgroups and joined by a second kernel.
 *   q        device, (B, Hq, head_dim) bfloat16 contiguous, 16-byte aligned
 *   cache    as filled by attn_kv_prepare for (B, S_cap, Hkv, head_dim): S_cap, B, Hkv and
 *            head_dim must be the values used there (they fix the cache's layout)
 *   cache_bytes  bytes of the cache allocation; below attn_fwd_workspace_bytes(B, S_cap, Hkv,
 *            head_dim, ATTN_DTYPE_BF16) the call returns ATTN_EWORKSPACE before any HIP call
 *   out      device, (B, Hq, head_dim) bfloat16, 16-byte aligned (written)
 *   lse      device, (B, Hq) float32, natural log (written)
 *   workspace  device, >= attn_decode_workspace_bytes(...) bytes, 16-byte aligned, caller owned
 *   0 <= q_pos < S_cap; Hq a multiple of Hkv
 * Returns ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EWORKSPACE or ATTN_EHIP as above.
 */
int attn_decode(const void *q, const void *cache, size_t cache_bytes, int B, int S_cap, int Hq,
                int Hkv, int head_dim, double rope_theta, int rope_style, int q_pos, void *out,
                float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode for a ragged batch, where each batch row has generated a different number of
 * tokens (the PaLM page's generation loop, section 2.7, run over a batch of sequences of
 * different lengths): batch row b's query sits at position q_pos[b] and attends to its own
 * cached keys 0 .. q_pos[b].  Arguments as for attn_decode, except
 *   q_pos    device, B int32 positions, 4-byte aligned, read by the kernel (so a serving loop
 *            can advance them on the GPU without a host round trip)
 *   max_pos  0 <= max_pos < S_cap, at least every q_pos[b]: it sizes the key ranges the work is
 *            split into; ranges past a row's position are empty.  A row whose q_pos[b] lies
 *            outside [0, max_pos] gets NaN in out and lse (checked on the GPU).
 * Returns the codes of attn_decode (ATTN_EINVAL also for a null or misaligned q_pos).
 */
int attn_decode_ragged(const void *q, const void *cache, size_t cache_bytes, int B, int S_cap,
                       int Hq, int Hkv, int head_dim, double rope_theta, int rope_style,
                       const int *q_pos, int max_pos, void *out, float *lse, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * Backward pass: the gradients dq, dk, dv of attn_fwd's out for a given output gradient dout
 * (the pages train these models -- PaLM-in-ColossalAI page, section 2.7, a cross-entropy
 * training loss -- and a training step needs them).  With P = softmax of the scaled, masked
 * scores of the rotated q and k, recomputed from the saved lse:
 *   dv = P^T dout (summed over the query heads sharing a K/V head),
 *   ds = P * (dout v^T - rowsum(dout * out)),
 *   dq = R^T (ds k' / sqrt(d)),  dk = R^T (ds^T q' / sqrt(d)) (summed like dv),
 * R the rotary rotation at each row's position.  The gradient of lse is taken as zero.
 *
 *   q, dout        device, (B, S, Hq, head_dim) bfloat16 contiguous, 16-byte aligned
 *   k, v           device, (B, S, Hkv, head_dim) bfloat16, 16-byte aligned
 *   out, lse       attn_fwd's outputs for the same q, k, v, rope_theta, rope_style, causal
 *   dq; dk, dv     device, shaped like q; like k (written), 16-byte aligned
 *   workspace      device, >= attn_bwd_workspace_bytes(...) bytes, 16-byte aligned (the
 *                  re-laid-out operands; for few (b, K/V head) pairs with many query heads
 *                  each, e.g. PaLM-540B's 48 heads on one K/V head, also fp32 partial dk and
 *                  dv of head splits, summed by a last kernel), caller owned
 * bf16 only; head_dim 64, 128 or 256 (at 256 the kernels keep the block that stays fixed over
 * their loop in LDS instead of registers).  Returns ATTN_OK, ATTN_EINVAL, ATTN_EUNSUPPORTED,
 * ATTN_EWORKSPACE or ATTN_EHIP with the meanings given for attn_fwd.
 */
size_t attn_bwd_workspace_bytes(int B, int S, int Hq, int Hkv, int head_dim);
int attn_bwd(const void *q, const void *k, const void *v, const void *out, const float *lse,
             const void *dout, int B, int S, int Hq, int Hkv, int head_dim, double rope_theta,
             int rope_style, int causal, void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes,
             void *stream);

/*
 * One step of the backward of ring attention (Picotron page, "context parallelism and ring
 * attention", where the ring is an autograd function): attn_bwd for queries at positions
 * q_pos0 .. q_pos0+S-1 against keys and values at k_pos0 .. k_pos0+S-1, with the visibility and
 * rotations of attn_fwd_shard.  out and lse must be the forward's results for these queries
 * over ALL key blocks (the merged ones, as attn_merge leaves them), so that the weights of this
 * block's keys are the full softmax's: P = exp(s - lse), 0 where masked.  The results are this
 * pair of blocks' parts of the gradients: dq summed over the key blocks a query block sees, and
 * dk, dv summed over the query blocks that see a key block, equal the gradients of the whole
 * sequence.  A row whose lse is -inf (it sees no key at all) contributes nothing.  attn_bwd is
 * this call with q_pos0 = k_pos0 = 0.
 *   q_pos0, k_pos0  >= 0, with q_pos0 + S and k_pos0 + S at most 2^30 (else ATTN_EINVAL)
 *   other arguments, workspace size and return codes as for attn_bwd
 */
int attn_bwd_shard(const void *q, const void *k, const void *v, const void *out, const float *lse,
                   const void *dout, int B, int S, int Hq, int Hkv, int head_dim, double rope_theta,
                   int rope_style, int causal, int q_pos0, int k_pos0, void *dq, void *dk, void *dv,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Timing events (hipEvent_t behind an opaque pointer).  create returns NULL on failure. */
void *attn_event_create(void);
int attn_event_destroy(void *ev);
/* Milliseconds between two recorded events; waits for `stop` to complete. */
int attn_event_elapsed_ms(void *start, void *stop, float *ms);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
