"""GPU parity of head_dim 256 (the PaLM page's 540B head size) against the float64 oracle.

head_dim 256 runs its own forward kernel (bf16 only) behind the same entry points; the
preparation pass, the shard offsets, both rotary forms and the lse merge are shared with the
other head sizes.  Tolerances as for the other bf16 tests: max-abs 2e-2 on out and lse.
"""

import numpy as np
import pytest
import torch

from oracle import attention, merge
from transformer_causal_attention_amd import AttnError, attn_fwd, attn_merge
from transformer_causal_attention_amd.workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print("[gpu-case]", *a, flush=True)


def np64(t):
    return t.double().numpy()


def w_of(B, S, Hq, Hkv, causal=True, theta=10000.0, seed=17):
    return Workload("d256", B, S, Hq, Hkv, 256, "bf16", 1.0, theta, causal, seed)


def check(out, lse, ref_o, ref_l, what):
    o = out.float().cpu().double().numpy()
    l = lse.cpu().double().numpy()
    seen = np.isfinite(ref_l)
    assert np.all(l[~seen] == -np.inf), f"{what}: rows without keys must have lse -inf"
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l[seen])), f"{what}: non-finite output"
    eo = np.abs(o - ref_o).max()
    el = np.abs(l[seen] - ref_l[seen]).max() if np.any(seen) else 0.0
    say(f"{what}: out err {eo:.3e}, lse err {el:.3e}")
    assert eo <= TOL and el <= TOL, what


SHAPES = [
    (1, 1, 4, 1, True), (2, 7, 2, 2, True), (1, 33, 8, 1, True), (1, 100, 4, 2, True), (2, 257, 6, 3, True),
    (1, 130, 3, 3, False), (2, 64, 8, 1, False),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}S{}H{}/{}{}".format(*s[:4], "c" if s[4] else "f"))
@pytest.mark.parametrize("interleaved", [False, True], ids=["half", "pairs"])
def test_small_shapes(shape, interleaved):
    B, S, Hq, Hkv, causal = shape
    w = w_of(B, S, Hq, Hkv, causal, seed=S + Hq)
    q, k, v = make_inputs(w)
    say(w, "interleaved", interleaved)
    out, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), w.rope_theta, causal, interleaved=interleaved)
    torch.cuda.synchronize()
    ref_o, ref_l = attention(np64(q), np64(k), np64(v), w.rope_theta, causal, interleaved=interleaved)
    check(out, lse, ref_o, ref_l, f"{w} interleaved {interleaved}")


def test_palm540b_heads_full_size():
    w = WORKLOADS["palm540b_d256"]
    q, k, v = make_inputs(w)
    say(w)
    out, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), w.rope_theta, w.causal)
    torch.cuda.synchronize()
    ref_o, ref_l = attention(np64(q), np64(k), np64(v), w.rope_theta, w.causal)
    check(out, lse, ref_o, ref_l, str(w))


def test_row0_is_exactly_v0():
    # row 0 sees only key 0: its weight is the exact maximum's 2^0 = 1, so out_0 = v_0 bit for bit
    w = w_of(1, 70, 4, 1, True, seed=3)
    q, k, v = make_inputs(w)
    out, _ = attn_fwd(q.cuda(), k.cuda(), v.cuda(), w.rope_theta, True)
    torch.cuda.synchronize()
    o = out.cpu()
    for h in range(w.Hq):
        assert torch.equal(o[:, 0, h], v[:, 0, 0]), f"head {h}"


def test_shard_offsets_and_ring_merge():
    # keys split into two shards at their positions, each attended with attn_fwd_shard and
    # joined by attn_merge, against the unsplit oracle
    w = w_of(1, 192, 8, 1, True, seed=29)
    q, k, v = make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for (qp, kp) in ((64, 0), (0, 40), (77, 13)):
        say(w, "q_pos0", qp, "k_pos0", kp)
        out, lse = attn_fwd(qd, kd, vd, w.rope_theta, True, q_pos0=qp, k_pos0=kp)
        torch.cuda.synchronize()
        ref_o, ref_l = attention(np64(q), np64(k), np64(v), w.rope_theta, True, q_pos0=qp, k_pos0=kp)
        check(out, lse, ref_o, ref_l, f"offsets ({qp}, {kp})")
    # queries 96..191 against key shards [0, 96) and [96, 192)
    n = 96
    q1 = qd[:, n:].contiguous()
    o_a, l_a = attn_fwd(q1, kd[:, :n].contiguous(), vd[:, :n].contiguous(), w.rope_theta, True, q_pos0=n, k_pos0=0)
    o_b, l_b = attn_fwd(q1, kd[:, n:].contiguous(), vd[:, n:].contiguous(), w.rope_theta, True, q_pos0=n, k_pos0=n)
    o_m, l_m = attn_merge(o_a, l_a, o_b, l_b)
    torch.cuda.synchronize()
    ref_o, ref_l = attention(np64(q), np64(k), np64(v), w.rope_theta, True)
    check(o_m, l_m, ref_o[:, n:], ref_l[:, :, n:], "two shards merged")
    # the merge kernel alone on the oracle's own parts
    ro_a, rl_a = attention(np64(q[:, n:]), np64(k[:, :n]), np64(v[:, :n]), w.rope_theta, True, q_pos0=n, k_pos0=0)
    ro_b, rl_b = attention(np64(q[:, n:]), np64(k[:, n:]), np64(v[:, n:]), w.rope_theta, True, q_pos0=n, k_pos0=n)
    mo, ml = merge(ro_a, rl_a, ro_b, rl_b)
    assert np.abs(mo - ref_o[:, n:]).max() < 1e-10


def test_fp32_rejected():
    w = w_of(1, 64, 4, 1, True)
    q, k, v = make_inputs(w)
    with pytest.raises(AttnError):
        attn_fwd(q.float().cuda(), k.float().cuda(), v.float().cuda(), w.rope_theta, True)
