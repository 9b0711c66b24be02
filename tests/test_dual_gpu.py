"""GPU parity of head_dim 64 grids large enough that the kernel gives each wave group a unit of
its own (two units per workgroup, one round of workgroups): more (unit, row-block pair) items
than CUs.  Covers MHA, GQA with 2 and 4 heads per group, an odd row-block count (a middle pair
whose two blocks are one), ragged sequences, no mask, both rotary forms and shard offsets,
against the float64 oracle with the bf16 tolerance 2e-2 on out and lse.
"""

import numpy as np
import pytest
import torch

from oracle import attention
from transformer_causal_attention_amd import attn_fwd
from transformer_causal_attention_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print("[gpu-case]", *a, flush=True)


def np64(t):
    return t.double().numpy()


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


# (B, S, Hq, Hkv): units = B * Hkv * G / hpw, rows per block 32 * 4 / hpw
SHAPES = [
    (3, 1000, 48, 48, True),   # MHA, 144 units x 4 pairs, ragged
    (8, 700, 16, 8, True),     # 2 heads per group: 64 units x 6 pairs, odd block count (11)
    (16, 512, 16, 4, True),    # 4 heads per group: 64 units x 8 pairs
    (4, 1024, 32, 32, False),  # MHA without the mask
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}S{}H{}/{}{}".format(*s[:4], "c" if s[4] else "f"))
@pytest.mark.parametrize("interleaved", [False, True], ids=["half", "pairs"])
def test_two_units_per_workgroup(shape, interleaved):
    B, S, Hq, Hkv, causal = shape
    w = Workload("dual", B, S, Hq, Hkv, 64, "bf16", 1.0, 10000.0, causal, S + Hq)
    q, k, v = make_inputs(w)
    say(w, "interleaved", interleaved)
    out, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), w.rope_theta, causal, interleaved=interleaved)
    torch.cuda.synchronize()
    ref_o, ref_l = attention(np64(q), np64(k), np64(v), w.rope_theta, causal, interleaved=interleaved)
    check(out, lse, ref_o, ref_l, f"{w} interleaved {interleaved}")


@pytest.mark.parametrize("offsets", [(128, 0), (0, 300), (700, 650)], ids=lambda o: f"q{o[0]}k{o[1]}")
def test_shard_offsets(offsets):
    qp, kp = offsets
    w = Workload("dual", 4, 640, 40, 40, 64, "bf16", 1.0, 10000.0, True, 31)
    q, k, v = make_inputs(w)
    say(w, "q_pos0", qp, "k_pos0", kp)
    out, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), w.rope_theta, True, q_pos0=qp, k_pos0=kp)
    torch.cuda.synchronize()
    ref_o, ref_l = attention(np64(q), np64(k), np64(v), w.rope_theta, True, q_pos0=qp, k_pos0=kp)
    check(out, lse, ref_o, ref_l, f"{w} offsets ({qp}, {kp})")


def test_row0_is_exactly_v0():
    w = Workload("dual", 4, 1024, 32, 32, 64, "bf16", 1.0, 10000.0, True, 4)
    q, k, v = make_inputs(w)
    out, _ = attn_fwd(q.cuda(), k.cuda(), v.cuda(), w.rope_theta, True)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu()[:, 0], v[:, 0])
