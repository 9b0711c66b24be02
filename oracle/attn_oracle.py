"""Float64 CPU oracle for causal self-attention with rotary positions and shared K/V heads.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct reference that the
GPU path is checked against.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path never calls it and shares no code with it.

Everything is computed in numpy float64 and follows the plain definition, step by step:

  1. rotary embedding (half-split "rotate_half" form) on q and k, never on v;
  2. scores = q_rot . k_rot^T / sqrt(head_dim);
  3. causal mask: a key later than the query gets -inf added to its score;
  4. softmax over keys with the row maximum subtracted first;
  5. out = softmax(scores) . v;
  6. lse = row max + ln(sum of exp(score - row max))  (natural log of the softmax denominator).

Sources (the pages this oracle follows):
  * Picotron page "Picotron model implementation: Llama architecture and Flash Attention
    integration", section 1 "embedding layer and positional encoding" -- apply_rotary_pos_emb
    with rotate_half = cat(-x2, x1) over the two halves of head_dim, x*cos + rotate_half*sin;
    section 2 "attention implementations" -- flash_attn_func(q, k, v, causal) on (B, S, H, D).
  * PaLM page "PaLM teaching implementation in ColossalAI", section 2.3 RotaryEmbedding --
    inv_freq = 1 / base^(arange(0, dim, 2) / dim), freqs = positions (outer) inv_freq,
    cat(freqs, freqs); applied to q and k only.  Section 2.5 Attention -- multi-query
    attention (one shared K/V head), causal mask on the upper triangle, row max subtracted
    before the softmax.
  * llama3-from-scratch page "parallel computing architecture": "attention score matrix"
    (q_rot @ k_rot.T / head_dim**0.5), "causal mask" (full(-inf) then triu(diagonal=1),
    added to the scores), "softmax" (over the key axis), "key-value sharing" (n_kv_heads=8
    for n_heads=32: every 4 query heads share one K/V head).

Readings where the pages are silent or disagree (each also listed in the design notes):
  * RoPE pairing: half-split (Picotron and PaLM pages) by default; with interleaved=True the
    llama3 page's adjacent pairs (2i, 2i+1), which it rotates as complex numbers.  The two are
    the same rotation under a fixed permutation of head_dim.
  * Positions are 0..S-1 for every batch row, unless a sequence shard passes its first
    query and key positions (q_pos0, k_pos0): queries then sit at q_pos0 + i and keys at
    k_pos0 + j, for the rotation and for the mask alike.  A query with no visible key has
    out = 0 and lse = -inf (an empty softmax denominator), so that merging it with another
    shard's partial result leaves that result unchanged.
  * GQA grouping is contiguous: query head h reads K/V head h // (Hq // Hkv).
  * lse is the natural-log logsumexp of the scaled scores over the visible keys.
  * The backward is the exact gradient of this forward with respect to q, k and v for a given
    gradient of the output (the pages train these models -- the PaLM page's wrapper returns a
    cross-entropy loss, section 2.7 -- but print no backward); the gradient of lse is not
    an input.
"""

import numpy as np

__all__ = [
    "rope_frequencies",
    "rope_angles",
    "rotate_half",
    "apply_rope",
    "apply_rope_interleaved",
    "causal_mask",
    "softmax_rows",
    "kv_head_of",
    "attention_weights",
    "attention",
    "merge",
    "attention_backward",
]


def rope_frequencies(head_dim, rope_theta):
    """Per-pair angular frequency theta_i = rope_theta ** (-2i / head_dim), i < head_dim/2.

    PaLM page, section 2.3 RotaryEmbedding: 1 / base ** (arange(0, dim, 2) / dim).
    The llama3 page builds the same numbers as 1 / rope_theta ** (arange(64) / 64) for
    head_dim 128.
    """
    i2 = np.arange(0, head_dim, 2, dtype=np.float64)
    return 1.0 / (np.float64(rope_theta) ** (i2 / np.float64(head_dim)))


def rope_angles(positions, head_dim, rope_theta):
    """Angle table (len(positions), head_dim): outer(positions, freqs) duplicated over both halves.

    PaLM page, section 2.3: freqs = positions x inv_freq, then cat((freqs, freqs), -1), so
    element c and element c + head_dim/2 share the angle of pair c.
    """
    freqs = np.outer(np.asarray(positions, dtype=np.float64), rope_frequencies(head_dim, rope_theta))
    return np.concatenate([freqs, freqs], axis=-1)


def rotate_half(x):
    """cat(-x2, x1) where x1, x2 are the first and second halves of the last axis.

    Picotron page, section 1 (apply_rotary_pos_emb).
    """
    half = x.shape[-1] // 2
    return np.concatenate([-x[..., half:], x[..., :half]], axis=-1)


def apply_rope(x, positions, rope_theta):
    """Rotate x of shape (B, len(positions), H, head_dim) by the angles of `positions`.

    Picotron page, section 1: x * cos + rotate_half(x) * sin, with cos/sin of the angle
    table broadcast over batch and heads.
    """
    x = np.asarray(x, dtype=np.float64)
    ang = rope_angles(positions, x.shape[-1], rope_theta)
    cos = np.cos(ang)[None, :, None, :]
    sin = np.sin(ang)[None, :, None, :]
    return x * cos + rotate_half(x) * sin


def apply_rope_interleaved(x, positions, rope_theta):
    """Rotate adjacent pairs (x_2i, x_2i+1) of x (B, len(positions), H, head_dim) by position x
    theta_i: x_2i' = x_2i cos - x_2i+1 sin, x_2i+1' = x_2i+1 cos + x_2i sin.

    llama3 page, "parallel rotation of queries and keys": the vector is split into adjacent
    pairs, each read as a complex number and multiplied by a unit complex number of angle
    position x theta_i, theta_i = rope_theta ** (-2i / head_dim) as for the half-split form.
    """
    x = np.asarray(x, dtype=np.float64)
    ang = np.outer(np.asarray(positions, dtype=np.float64), rope_frequencies(x.shape[-1], rope_theta))
    cos = np.cos(ang)[None, :, None, :]
    sin = np.sin(ang)[None, :, None, :]
    ev, od = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = ev * cos - od * sin
    out[..., 1::2] = od * cos + ev * sin
    return out


def causal_mask(query_positions, n_keys, key_pos0=0):
    """Additive mask (len(query_positions), n_keys): 0 where the key's position is at most the
    query's, -inf where it is later.  Key j sits at position key_pos0 + j.

    llama3 page, "causal mask": full(-inf) followed by triu(diagonal=1), added to the scores.
    Written for an arbitrary set of query positions so single rows can be evaluated alone.
    """
    j = key_pos0 + np.arange(n_keys)
    i = np.asarray(query_positions)
    return np.where(j[None, :] > i[:, None], -np.inf, 0.0)


def softmax_rows(scores):
    """Numerically stable softmax along the last axis; also returns the row max and row sum.

    PaLM page, section 2.5: subtract the row maximum, then softmax.
    Returns (P, m, l) with P = exp(scores - m) / l, m = row max, l = sum exp(scores - m).
    A row whose every score is -inf (no visible key) has P = 0, m = -inf and l = 0.
    """
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - np.where(np.isfinite(m), m, 0.0))
    l = e.sum(axis=-1, keepdims=True)
    return e / np.where(l > 0, l, 1.0), m[..., 0], l[..., 0]


def kv_head_of(h, n_q_heads, n_kv_heads):
    """K/V head read by query head h: contiguous groups of Hq/Hkv query heads.

    llama3 page, "key-value sharing": every 4 query heads share one K/V head (32 over 8);
    PaLM page, section 2.5: a single K/V head shared by every query head.
    """
    if n_q_heads % n_kv_heads != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    return h // (n_q_heads // n_kv_heads)


def attention_weights(q_rot, k_rot, query_positions, causal, key_pos0=0):
    """Softmax weights for one (batch, head): q_rot (R, d) at query_positions, k_rot (S, d)
    at positions key_pos0 + j.

    llama3 page, "attention score matrix": scores = q_rot @ k_rot.T / head_dim ** 0.5;
    "causal mask": add the mask; "softmax": over the key axis.
    Returns (P, m, l) as softmax_rows does.
    """
    d = q_rot.shape[-1]
    scores = (q_rot @ k_rot.T) / np.sqrt(np.float64(d))
    if causal:
        scores = scores + causal_mask(query_positions, k_rot.shape[0], key_pos0)
    return softmax_rows(scores)


def attention(q, k, v, rope_theta, causal=True, rows=None, q_pos0=0, k_pos0=0, interleaved=False):
    """Causal (or full) RoPE attention with shared K/V heads, in float64.

    q: (B, S, Hq, d); k, v: (B, S, Hkv, d); Hq a multiple of Hkv; d even.
    rows: optional 1-D array of query rows to evaluate (default: all S rows).  Each output row
    depends only on its own query and the keys, so evaluating a subset is the same definition
    restricted to those rows.
    q_pos0, k_pos0: positions of query row 0 and key row 0 (a sequence shard's offsets; the
    Picotron page's ring attention passes K/V blocks of other positions around the ranks).
    interleaved: rotate adjacent pairs (llama3 page) instead of the two halves.

    Returns (out, lse): out (B, R, Hq, d) float64 and lse (B, Hq, R) float64, R = len(rows).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be (B, S, Hkv, d) with q's B, S and d")
    if d % 2 != 0:
        raise ValueError("head_dim must be even for the half-split rotation")
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)

    q_positions = q_pos0 + rows
    rope = apply_rope_interleaved if interleaved else apply_rope
    q_rot = rope(q[:, rows], q_positions, rope_theta)
    k_rot = rope(k, k_pos0 + np.arange(S), rope_theta)

    out = np.empty((B, len(rows), Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq, len(rows)), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            P, m, l = attention_weights(q_rot[b, :, h, :], k_rot[b, :, g, :], q_positions, causal, k_pos0)
            out[b, :, h, :] = P @ v[b, :, g, :]
            with np.errstate(divide="ignore"):
                lse[b, h, :] = m + np.log(l)  # -inf for a row with no visible key
    return out, lse


def merge(o1, lse1, o2, lse2):
    """Join two partial results over disjoint key sets: lse = logaddexp(lse1, lse2) and
    out = exp(lse1 - lse) * o1 + exp(lse2 - lse) * o2 (a row empty in both stays empty).

    This is the combination ring attention performs when each rank has attended to one block
    of keys (Picotron page, context parallelism and ring attention); with lse the natural-log
    softmax denominator of each part it reproduces attention over the union of the keys.
    o: (B, R, H, d); lse: (B, H, R).
    """
    lse1 = np.asarray(lse1, dtype=np.float64)
    lse2 = np.asarray(lse2, dtype=np.float64)
    lse = np.logaddexp(lse1, lse2)
    safe = np.where(np.isfinite(lse), lse, 0.0)
    w1 = np.where(np.isfinite(lse), np.exp(lse1 - safe), 0.0)
    w2 = np.where(np.isfinite(lse), np.exp(lse2 - safe), 0.0)
    # (B, H, R) weights onto (B, R, H, d) rows
    out = (np.transpose(w1, (0, 2, 1))[..., None] * np.asarray(o1, dtype=np.float64)
           + np.transpose(w2, (0, 2, 1))[..., None] * np.asarray(o2, dtype=np.float64))
    return out, lse


def attention_backward(q, k, v, dout, rope_theta, causal=True, interleaved=False):
    """Gradients (dq, dk, dv) of the attention above for an output gradient dout, in float64.

    q, dout: (B, S, Hq, d); k, v: (B, S, Hkv, d).  Differentiating the forward's steps in
    reverse order, for each (batch, query head h) with K/V head g:
      out = P v                 ->  dv_g += P^T dout,   dP = dout v^T
      P = softmax(s) per row    ->  ds = P * (dP - rowsum(dout * out))
      s = q' k'^T / sqrt(d)     ->  dq' = ds k' / sqrt(d),   dk'_g += ds^T q' / sqrt(d)
      x' = R(position) x        ->  dx = R(position)^T dx' = R(-position) dx'
    (masked scores have P = 0 and so no gradient; a K/V head's gradient sums over the query
    heads that share it).
    interleaved: the adjacent-pair rotation, as in attention().
    Returns dq (B, S, Hq, d), dk and dv (B, S, Hkv, d).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, d) or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("k, v must be (B, S, Hkv, d) and dout like q")
    pos = np.arange(S)
    rope = apply_rope_interleaved if interleaved else apply_rope
    q_rot = rope(q, pos, rope_theta)
    k_rot = rope(k, pos, rope_theta)
    scale = 1.0 / np.sqrt(np.float64(d))

    dq_rot = np.zeros_like(q_rot)
    dk_rot = np.zeros_like(k_rot)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            P, _, _ = attention_weights(q_rot[b, :, h, :], k_rot[b, :, g, :], pos, causal)
            o = P @ v[b, :, g, :]
            do = dout[b, :, h, :]
            dv[b, :, g, :] += P.T @ do
            dP = do @ v[b, :, g, :].T
            ds = P * (dP - (do * o).sum(axis=-1, keepdims=True))
            dq_rot[b, :, h, :] = (ds @ k_rot[b, :, g, :]) * scale
            dk_rot[b, :, g, :] += (ds.T @ q_rot[b, :, h, :]) * scale
    dq = rope(dq_rot, -pos, rope_theta)
    dk = rope(dk_rot, -pos, rope_theta)
    return dq, dk, dv


def attention_backward_shard(q, k, v, dout, out, lse, rope_theta, causal=True, q_pos0=0, k_pos0=0,
                             interleaved=False):
    """The part of the gradients that one block of keys contributes, for one block of queries,
    given the finished forward of those queries over every key block: one step of the backward
    of ring attention, which the Picotron page runs as an autograd function ("context
    parallelism and ring attention"; the pages print no backward, so this is the derivative of
    the definition restricted to one key block).

    q, dout: (B, S, Hq, d) at query positions q_pos0 + i; k, v: (B, S, Hkv, d) at key positions
    k_pos0 + j; out (B, S, Hq, d) and lse (B, Hq, S): the forward's results for these queries
    over all keys (for one block alone, attention()'s own).  With the weights of this block's
    keys taken from the whole softmax, P = exp(s - lse) (0 where masked, and for a row whose lse
    is -inf), the chain rule of out = sum over blocks of P v gives
      dv_g += P^T dout,   dP = dout v^T,   ds = P * (dP - rowsum(dout * out)),
      dq' = ds k' / sqrt(d),   dk'_g += ds^T q' / sqrt(d),   dx = R(-position) dx'.
    Summed over key blocks, dq is the full dq; summed over query blocks, dk and dv are.
    Returns dq (B, S, Hq, d), dk and dv (B, S, Hkv, d).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, d) or v.shape != k.shape or dout.shape != q.shape or out.shape != q.shape:
        raise ValueError("k, v must be (B, S, Hkv, d); dout and out like q")
    if lse.shape != (B, Hq, S):
        raise ValueError("lse must be (B, Hq, S)")
    q_positions = q_pos0 + np.arange(S)
    k_positions = k_pos0 + np.arange(S)
    rope = apply_rope_interleaved if interleaved else apply_rope
    q_rot = rope(q, q_positions, rope_theta)
    k_rot = rope(k, k_positions, rope_theta)
    scale = 1.0 / np.sqrt(np.float64(d))

    dq_rot = np.zeros_like(q_rot)
    dk_rot = np.zeros_like(k_rot)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            scores = (q_rot[b, :, h, :] @ k_rot[b, :, g, :].T) * scale
            if causal:
                scores = scores + causal_mask(q_positions, S, k_pos0)
            L = lse[b, h, :][:, None]
            with np.errstate(invalid="ignore"):
                P = np.where(np.isfinite(L) & np.isfinite(scores), np.exp(scores - np.where(np.isfinite(L), L, 0.0)),
                             0.0)
            do = dout[b, :, h, :]
            dv[b, :, g, :] += P.T @ do
            dP = do @ v[b, :, g, :].T
            ds = P * (dP - (do * out[b, :, h, :]).sum(axis=-1, keepdims=True))
            dq_rot[b, :, h, :] = (ds @ k_rot[b, :, g, :]) * scale
            dk_rot[b, :, g, :] += (ds.T @ q_rot[b, :, h, :]) * scale
    dq = rope(dq_rot, -q_positions, rope_theta)
    dk = rope(dk_rot, -k_positions, rope_theta)
    return dq, dk, dv
