"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch every one.

Each mutation replaces one oracle function by a subtly wrong version -- a dropped term, a
wrong sign or index, a transposed operand, an off-by-one -- and the test asserts that at
least one pin in oracle_pins fails.  This is what shows the pins constrain the oracle.
"""

import numpy as np
import pytest

import oracle_pins
from oracle import attn_oracle as O


def _rotate_half_wrong_sign(x):
    half = x.shape[-1] // 2
    return np.concatenate([x[..., half:], -x[..., :half]], axis=-1)


def _rotate_half_swapped_halves(x):
    half = x.shape[-1] // 2
    return np.concatenate([-x[..., :half], x[..., half:]], axis=-1)


def _freq_missing_two(head_dim, rope_theta):
    i = np.arange(0, head_dim // 2, dtype=np.float64)
    return 1.0 / (np.float64(rope_theta) ** (i / head_dim))


def _freq_wrong_sign(head_dim, rope_theta):
    i2 = np.arange(0, head_dim, 2, dtype=np.float64)
    return np.float64(rope_theta) ** (i2 / head_dim)


def _angles_interleaved_dup(positions, head_dim, rope_theta):
    freqs = np.outer(np.asarray(positions, dtype=np.float64), O.rope_frequencies(head_dim, rope_theta))
    return np.repeat(freqs, 2, axis=-1)


def _apply_rope_cos_sin_swapped(x, positions, rope_theta):
    x = np.asarray(x, dtype=np.float64)
    ang = O.rope_angles(positions, x.shape[-1], rope_theta)
    return x * np.sin(ang)[None, :, None, :] + O.rotate_half(x) * np.cos(ang)[None, :, None, :]


def _apply_rope_positions_plus_one(x, positions, rope_theta):
    x = np.asarray(x, dtype=np.float64)
    ang = O.rope_angles(np.asarray(positions) + 1, x.shape[-1], rope_theta)
    return x * np.cos(ang)[None, :, None, :] + O.rotate_half(x) * np.sin(ang)[None, :, None, :]


def _mask_includes_diagonal(query_positions, n_keys, key_pos0=0):
    j = key_pos0 + np.arange(n_keys)
    i = np.asarray(query_positions)
    return np.where(j[None, :] >= i[:, None], -np.inf, 0.0)


def _mask_reversed(query_positions, n_keys, key_pos0=0):
    j = key_pos0 + np.arange(n_keys)
    i = np.asarray(query_positions)
    return np.where(j[None, :] < i[:, None], -np.inf, 0.0)


def _mask_off_by_one(query_positions, n_keys, key_pos0=0):
    j = key_pos0 + np.arange(n_keys)
    i = np.asarray(query_positions)
    return np.where(j[None, :] > i[:, None] + 1, -np.inf, 0.0)


def _mask_ignores_key_offset(query_positions, n_keys, key_pos0=0):
    j = np.arange(n_keys)
    i = np.asarray(query_positions)
    return np.where(j[None, :] > i[:, None], -np.inf, 0.0)


def _softmax_no_empty_guard(scores):
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    l = e.sum(axis=-1, keepdims=True)
    return e / l, m[..., 0], l[..., 0]


def _merge_weights_swapped(o1, lse1, o2, lse2):
    lse = np.logaddexp(lse1, lse2)
    w1 = np.exp(np.asarray(lse2) - lse)
    w2 = np.exp(np.asarray(lse1) - lse)
    return (np.transpose(w1, (0, 2, 1))[..., None] * o1 + np.transpose(w2, (0, 2, 1))[..., None] * o2), lse


def _merge_plain_average(o1, lse1, o2, lse2):
    return 0.5 * (np.asarray(o1) + np.asarray(o2)), np.logaddexp(lse1, lse2)


def _softmax_wrong_axis(scores):
    m = scores.max(axis=0, keepdims=True)
    e = np.exp(scores - m)
    l = e.sum(axis=0, keepdims=True)
    P = e / l
    mm = scores.max(axis=-1)
    return P, mm, np.exp(scores - mm[:, None]).sum(-1)


def _softmax_no_normalise(scores):
    m = scores.max(axis=-1, keepdims=True)
    e = np.exp(scores - m)
    l = e.sum(axis=-1, keepdims=True)
    return e, m[..., 0], l[..., 0]


def _kv_head_modulo(h, n_q_heads, n_kv_heads):
    return h % n_kv_heads


def _weights_scale_by_d(q_rot, k_rot, query_positions, causal, key_pos0=0):
    d = q_rot.shape[-1]
    scores = (q_rot @ k_rot.T) / np.float64(d)
    if causal:
        scores = scores + O.causal_mask(query_positions, k_rot.shape[0], key_pos0)
    return O.softmax_rows(scores)


def _weights_no_scale(q_rot, k_rot, query_positions, causal, key_pos0=0):
    scores = q_rot @ k_rot.T
    if causal:
        scores = scores + O.causal_mask(query_positions, k_rot.shape[0], key_pos0)
    return O.softmax_rows(scores)


def _weights_ignore_causal(q_rot, k_rot, query_positions, causal, key_pos0=0):
    d = q_rot.shape[-1]
    return O.softmax_rows((q_rot @ k_rot.T) / np.sqrt(np.float64(d)))


def _attention_variant(*, lse_drops_max=False, rope_v=False, transpose_p=False, unrotated_k=False,
                       k_rope_no_offset=False, q_rope_no_offset=False):
    def attention(q, k, v, rope_theta, causal=True, rows=None, q_pos0=0, k_pos0=0, interleaved=False):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        B, S, Hq, d = q.shape
        Hkv = k.shape[2]
        rows = np.arange(S) if rows is None else np.asarray(rows)
        qp = rows + (0 if q_rope_no_offset else q_pos0)
        rope = O.apply_rope_interleaved if interleaved else O.apply_rope
        q_rot = rope(q[:, rows], qp, rope_theta)
        kp = np.arange(S) + (0 if k_rope_no_offset else k_pos0)
        k_rot = k if unrotated_k else rope(k, kp, rope_theta)
        vv = O.apply_rope(v, np.arange(S), rope_theta) if rope_v else v
        out = np.empty((B, len(rows), Hq, d))
        lse = np.empty((B, Hq, len(rows)))
        for b in range(B):
            for h in range(Hq):
                g = O.kv_head_of(h, Hq, Hkv)
                P, m, l = O.attention_weights(q_rot[b, :, h], k_rot[b, :, g], q_pos0 + rows, causal, k_pos0)
                if transpose_p and P.shape[0] == P.shape[1]:
                    P = P.T
                out[b, :, h] = P @ vv[b, :, g]
                with np.errstate(divide="ignore"):
                    lse[b, h] = np.log(l) if lse_drops_max else m + np.log(l)
        return out, lse

    return attention


def _backward_variant(*, drop_rowsum=False, rope_forward_sign=False, no_scale=False, ds_untransposed=False,
                      dv_untransposed=False, rowsum_of_dp=False):
    def attention_backward(q, k, v, dout, rope_theta, causal=True, interleaved=False):
        q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
        B, S, Hq, d = q.shape
        Hkv = k.shape[2]
        pos = np.arange(S)
        rope = O.apply_rope_interleaved if interleaved else O.apply_rope
        q_rot, k_rot = rope(q, pos, rope_theta), rope(k, pos, rope_theta)
        scale = 1.0 if no_scale else 1.0 / np.sqrt(np.float64(d))
        dq_rot, dk_rot, dv = np.zeros_like(q_rot), np.zeros_like(k_rot), np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                g = O.kv_head_of(h, Hq, Hkv)
                P, _, _ = O.attention_weights(q_rot[b, :, h], k_rot[b, :, g], pos, causal)
                o = P @ v[b, :, g]
                do = dout[b, :, h]
                dv[b, :, g] += (P if dv_untransposed else P.T) @ do
                dP = do @ v[b, :, g].T
                if drop_rowsum:
                    ds = P * dP
                elif rowsum_of_dp:
                    ds = P * (dP - dP.sum(axis=-1, keepdims=True))
                else:
                    ds = P * (dP - (do * o).sum(axis=-1, keepdims=True))
                dq_rot[b, :, h] = (ds @ k_rot[b, :, g]) * scale
                dk_rot[b, :, g] += ((ds if ds_untransposed else ds.T) @ q_rot[b, :, h]) * scale
        back = pos if rope_forward_sign else -pos
        return rope(dq_rot, back, rope_theta), rope(dk_rot, back, rope_theta), dv

    return attention_backward


def _shard_backward_variant(*, mask_no_key_offset=False, dq_back_no_offset=False, dk_back_no_offset=False,
                            block_softmax=False):
    def attention_backward_shard(q, k, v, dout, out, lse, rope_theta, causal=True, q_pos0=0, k_pos0=0,
                                 interleaved=False):
        q, k, v, dout, out, lse = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout, out, lse))
        B, S, Hq, d = q.shape
        Hkv = k.shape[2]
        qp, kp = q_pos0 + np.arange(S), k_pos0 + np.arange(S)
        rope = O.apply_rope_interleaved if interleaved else O.apply_rope
        q_rot, k_rot = rope(q, qp, rope_theta), rope(k, kp, rope_theta)
        scale = 1.0 / np.sqrt(np.float64(d))
        dq_rot, dk_rot, dv = np.zeros_like(q_rot), np.zeros_like(k_rot), np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                g = O.kv_head_of(h, Hq, Hkv)
                sc = (q_rot[b, :, h] @ k_rot[b, :, g].T) * scale
                if causal:
                    sc = sc + O.causal_mask(qp, S, 0 if mask_no_key_offset else k_pos0)
                if block_softmax:
                    P, _, _ = O.softmax_rows(sc)
                else:
                    L = lse[b, h][:, None]
                    with np.errstate(invalid="ignore"):
                        P = np.where(np.isfinite(L) & np.isfinite(sc), np.exp(sc - np.where(np.isfinite(L), L, 0.0)),
                                     0.0)
                do = dout[b, :, h]
                dv[b, :, g] += P.T @ do
                ds = P * (do @ v[b, :, g].T - (do * out[b, :, h]).sum(axis=-1, keepdims=True))
                dq_rot[b, :, h] = (ds @ k_rot[b, :, g]) * scale
                dk_rot[b, :, g] += (ds.T @ q_rot[b, :, h]) * scale
        dq = rope(dq_rot, -(np.arange(S) if dq_back_no_offset else qp), rope_theta)
        dk = rope(dk_rot, -(np.arange(S) if dk_back_no_offset else kp), rope_theta)
        return dq, dk, dv

    return attention_backward_shard


def _rope_interleaved_half_split(x, positions, rope_theta):
    return O.apply_rope(x, positions, rope_theta)


def _rope_interleaved_sign(x, positions, rope_theta):
    x = np.asarray(x, dtype=np.float64)
    ang = np.outer(np.asarray(positions, dtype=np.float64), O.rope_frequencies(x.shape[-1], rope_theta))
    c, s_ = np.cos(ang)[None, :, None, :], np.sin(ang)[None, :, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s_
    out[..., 1::2] = x[..., 1::2] * c - x[..., 0::2] * s_
    return out


MUTATIONS = {
    "rotate_half_wrong_sign": ("rotate_half", _rotate_half_wrong_sign),
    "rotate_half_swapped_halves": ("rotate_half", _rotate_half_swapped_halves),
    "frequencies_missing_factor_two": ("rope_frequencies", _freq_missing_two),
    "frequencies_wrong_sign": ("rope_frequencies", _freq_wrong_sign),
    "angles_interleaved_duplication": ("rope_angles", _angles_interleaved_dup),
    "rope_cos_sin_swapped": ("apply_rope", _apply_rope_cos_sin_swapped),
    "rope_positions_off_by_one": ("apply_rope", _apply_rope_positions_plus_one),
    "mask_includes_diagonal": ("causal_mask", _mask_includes_diagonal),
    "mask_reversed": ("causal_mask", _mask_reversed),
    "mask_off_by_one": ("causal_mask", _mask_off_by_one),
    "softmax_wrong_axis": ("softmax_rows", _softmax_wrong_axis),
    "softmax_not_normalised": ("softmax_rows", _softmax_no_normalise),
    "gqa_modulo_grouping": ("kv_head_of", _kv_head_modulo),
    "scale_one_over_d": ("attention_weights", _weights_scale_by_d),
    "scale_dropped": ("attention_weights", _weights_no_scale),
    "causal_flag_ignored": ("attention_weights", _weights_ignore_causal),
    "lse_drops_row_max": ("attention", _attention_variant(lse_drops_max=True)),
    "rope_applied_to_v": ("attention", _attention_variant(rope_v=True)),
    "weights_transposed": ("attention", _attention_variant(transpose_p=True)),
    "k_left_unrotated": ("attention", _attention_variant(unrotated_k=True)),
    "mask_ignores_key_offset": ("causal_mask", _mask_ignores_key_offset),
    "empty_rows_unguarded": ("softmax_rows", _softmax_no_empty_guard),
    "k_rotation_ignores_offset": ("attention", _attention_variant(k_rope_no_offset=True)),
    "q_rotation_ignores_offset": ("attention", _attention_variant(q_rope_no_offset=True)),
    "merge_weights_swapped": ("merge", _merge_weights_swapped),
    "merge_plain_average": ("merge", _merge_plain_average),
    "backward_drops_rowsum": ("attention_backward", _backward_variant(drop_rowsum=True)),
    "backward_rowsum_of_dp": ("attention_backward", _backward_variant(rowsum_of_dp=True)),
    "backward_rope_not_inverted": ("attention_backward", _backward_variant(rope_forward_sign=True)),
    "backward_scale_dropped": ("attention_backward", _backward_variant(no_scale=True)),
    "backward_dk_untransposed": ("attention_backward", _backward_variant(ds_untransposed=True)),
    "backward_dv_untransposed": ("attention_backward", _backward_variant(dv_untransposed=True)),
    "shard_backward_mask_ignores_key_offset": ("attention_backward_shard",
                                               _shard_backward_variant(mask_no_key_offset=True)),
    "shard_backward_dq_rotated_back_at_row": ("attention_backward_shard",
                                              _shard_backward_variant(dq_back_no_offset=True)),
    "shard_backward_dk_rotated_back_at_row": ("attention_backward_shard",
                                              _shard_backward_variant(dk_back_no_offset=True)),
    "shard_backward_block_softmax": ("attention_backward_shard", _shard_backward_variant(block_softmax=True)),
    "interleaved_is_half_split": ("apply_rope_interleaved", _rope_interleaved_half_split),
    "interleaved_wrong_sign": ("apply_rope_interleaved", _rope_interleaved_sign),
}


def _failing_pins():
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:  # AssertionError, or a crash the slip causes
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = _failing_pins()
    assert failed, f"mutation {name} passed every pin"


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []
