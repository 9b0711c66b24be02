"""GPU parity of the decode step (attn_kv_prepare + attn_decode) against the float64 oracle.

A decode query at position q_pos attends to keys 0 .. q_pos: it is row q_pos of causal
attention, so the oracle is attention(q, k, v, rope_theta, causal=True, rows=[q_pos]) with the
decode query placed at row q_pos.  Tolerance as for the bf16 forward: 2e-2 on out and lse.
"""

import numpy as np
import pytest
import torch

from oracle import attention
from transformer_causal_attention_amd import attn_decode, attn_fwd, decode_workspace_bytes, kv_prepare, new_kv_cache
from transformer_causal_attention_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print("[gpu-case]", *a, flush=True)


def w_of(B, S, Hq, Hkv, d, theta=10000.0, sigma=1.0, seed=3):
    return Workload("decode", B, S, Hq, Hkv, d, "bf16", sigma, theta, True, seed)


def check_row(q, k, v, w, pos, out, lse, what):
    """out (B, Hq, d), lse (B, Hq) against row pos of the oracle."""
    ref_o, ref_l = attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.rope_theta, True,
                             rows=[pos])
    o = out.float().cpu().double().numpy()
    l = lse.cpu().double().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), what
    eo = np.abs(o - ref_o[:, 0]).max()
    el = np.abs(l - ref_l[:, :, 0]).max()
    say(f"{what}: out err {eo:.3e}, lse err {el:.3e}")
    assert eo <= TOL and el <= TOL, what


def poisoned_cache(w):
    c = new_kv_cache(w.B, w.S, w.Hkv, w.d, "cuda")
    c.fill_(0xFF)  # bf16 0xFFFF is a NaN: any read of an unprepared tile would show
    return c


SHAPES = [
    (1, 2048, 32, 8, 128, 500000.0),  # Llama-3-8B heads
    (8, 1024, 8, 1, 64, 10000.0),     # multi-query, PaLM-style heads
    (4, 1024, 32, 32, 64, 10000.0),   # multi-head
    (2, 300, 8, 2, 128, 10000.0),     # ragged capacity
    (1, 200, 128, 2, 64, 10000.0),    # 64 heads per K/V head: two head blocks
    (3, 130, 40, 1, 128, 10000.0),    # 40 heads on one K/V head: a partial head block
    (2, 1500, 48, 1, 256, 10000.0),   # PaLM-540B heads: 48 on one K/V head, head_dim 256
    (2, 300, 8, 2, 256, 10000.0),     # head_dim 256, grouped
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}S{}H{}/{}d{}".format(*s[:5]))
def test_decode_positions(shape):
    B, S, Hq, Hkv, d, theta = shape
    w = w_of(B, S, Hq, Hkv, d, theta, seed=S + Hq)
    q, k, v = make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cache = poisoned_cache(w)
    kv_prepare(kd, vd, theta, 0, S, cache)
    for pos in sorted({0, 1, 63, 64, 65, S // 2, S - 2, S - 1}):
        say(w, "q_pos", pos)
        out, lse = attn_decode(qd[:, pos].contiguous(), cache, S, Hkv, theta, pos)
        torch.cuda.synchronize()
        check_row(q, k, v, w, pos, out, lse, f"{w} q_pos {pos}")


def test_decode_incremental_append():
    """Keys appended one at a time (each call re-prepares only the newest tile) with the rows
    past the newest key still NaN in k, v and the cache, decoded after every append."""
    B, S, Hq, Hkv, d = 2, 192, 16, 4, 128
    w = w_of(B, S, Hq, Hkv, d, seed=11)
    q, k, v = make_inputs(w)
    kd = torch.full_like(k, float("nan")).cuda()
    vd = torch.full_like(v, float("nan")).cuda()
    qd = q.cuda()
    cache = poisoned_cache(w)
    n0 = 60
    kd[:, :n0] = k[:, :n0].cuda()
    vd[:, :n0] = v[:, :n0].cuda()
    kv_prepare(kd, vd, w.rope_theta, 0, n0, cache)
    for pos in range(n0, 140):
        kd[:, pos] = k[:, pos].cuda()
        vd[:, pos] = v[:, pos].cuda()
        kv_prepare(kd, vd, w.rope_theta, pos, pos + 1, cache)
        out, lse = attn_decode(qd[:, pos].contiguous(), cache, S, Hkv, w.rope_theta, pos)
        if pos in (n0, 63, 64, 65, 100, 127, 128, 139):
            torch.cuda.synchronize()
            say(w, "appended through", pos)
            check_row(q, k, v, w, pos, out, lse, f"{w} append {pos}")


@pytest.mark.parametrize("d", [64, 256])
def test_decode_matches_forward_rows(d):
    """Decode at every position of a short sequence equals the forward's rows (both bf16
    paths against each other, within twice the oracle tolerance)."""
    B, S, Hq, Hkv = 1, 130, 8, 2
    w = w_of(B, S, Hq, Hkv, d, seed=21)
    q, k, v = make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    fo, fl = attn_fwd(qd, kd, vd, w.rope_theta, True)
    cache = new_kv_cache(B, S, Hkv, d, "cuda")
    kv_prepare(kd, vd, w.rope_theta, 0, S, cache)
    ws = torch.empty(decode_workspace_bytes(B, Hq, Hkv, d), dtype=torch.uint8, device="cuda")
    worst = 0.0
    for pos in range(S):
        out, lse = attn_decode(qd[:, pos].contiguous(), cache, S, Hkv, w.rope_theta, pos, workspace=ws)
        worst = max(worst, (out.float() - fo[:, pos].float()).abs().max().item(),
                    (lse - fl[:, :, pos]).abs().max().item())
    torch.cuda.synchronize()
    say("decode vs forward rows, worst", worst)
    assert worst <= 2 * TOL


@pytest.mark.parametrize("d", [64, 128, 256])
def test_decode_staircase_scores(d):
    """Every 64-key tile scores about 68 (natural units) above the one before, so each tile and
    each key split is rescaled by its successor.  Inputs sit in the lowest-frequency rotation
    pair, which barely turns at rope_theta 5e5.  lse is checked to 2e-2 + 2^-8 * |s| as for
    the forward: the bf16 rounding of the scaled query moves a score s by up to 2^-9 |s|."""
    B, S, Hq, Hkv = 1, 700, 8, 1
    w = w_of(B, S, Hq, Hkv, d, theta=500000.0, seed=31 + d)
    q, k, v = (t.float() for t in make_inputs(w))
    c, c2 = d // 2 - 1, d - 1
    q, k = 0.25 * q, 0.25 * k
    q[..., c] = 68.0 * d ** 0.5 / 8.0
    q[..., c2] = 0.0
    k[..., c2] = 0.0
    k[..., c] = 8.0 * (torch.arange(S) // 64).float()[None, :, None]
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cache = poisoned_cache(w)
    kv_prepare(kd, vd, w.rope_theta, 0, S, cache)
    for pos in (5, 64, 350, 699):
        out, lse = attn_decode(qd[:, pos].contiguous(), cache, S, Hkv, w.rope_theta, pos)
        torch.cuda.synchronize()
        ref_o, ref_l = attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.rope_theta, True,
                                 rows=[pos])
        o = out.float().cpu().double().numpy()
        eo = np.abs(o - ref_o[:, 0]).max()
        el = np.abs(lse.cpu().double().numpy() - ref_l[:, :, 0])
        tol_l = 2e-2 + 2.0 ** -8 * (np.abs(ref_l[:, :, 0]) + np.log(S))
        say(f"staircase d{d} q_pos {pos}: out err {eo:.3e}, lse err {el.max():.3e} (tol up to {tol_l.max():.3e})")
        assert np.all(np.isfinite(o)) and eo <= TOL
        assert np.all(el <= tol_l)
