"""GPU parity of the sequence-shard entry points against the float64 oracle.

attn_fwd_shard (attn_fwd with q_pos0 / k_pos0): queries at q_pos0 + i, keys at k_pos0 + j, for
the rotation and the causal mask; rows that see no key give out 0 and lse -inf exactly.
attn_merge: lse = logaddexp(lse1, lse2), out = e^(lse1-lse) o1 + e^(lse2-lse) o2.
Composed, they evaluate causal attention over a sequence split into shards (one ring-attention
pass on one GPU), which must match the unsharded oracle.  Tolerances as in test_parity_gpu.
"""

import numpy as np
import pytest
import torch

from oracle import attention, merge
from transformer_causal_attention_amd import attn_fwd, attn_merge
from transformer_causal_attention_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def say(*a):
    print("[gpu-case]", *a, flush=True)


def compare(dtype, out, lse, ref_out, ref_lse, what):
    o = out.float().cpu().double().numpy()
    l = lse.cpu().double().numpy()
    empty = ~np.isfinite(ref_lse)  # (B, H, R): rows that see no key
    assert np.all(l[empty] == -np.inf), f"{what}: empty rows must have lse -inf"
    assert np.all(np.isfinite(l[~empty])), f"{what}: non-finite lse on a row with keys"
    e_rows = np.transpose(empty, (0, 2, 1))  # (B, R, H)
    assert np.all(o[e_rows] == 0.0), f"{what}: empty rows must have out 0"
    assert np.all(np.isfinite(o)), f"{what}: non-finite out"
    eo = np.abs(o - ref_out).max()
    el = np.abs(l[~empty] - ref_lse[~empty]).max() if np.any(~empty) else 0.0
    say(f"{what}: out err {eo:.3e}, lse err {el:.3e}, empty rows {int(empty.sum())}")
    assert eo <= TOL[dtype] and el <= TOL[dtype], what


def w_of(B, S, Hq, Hkv, d, dtype, causal=True, seed=5):
    return Workload("shard", B, S, Hq, Hkv, d, dtype, 1.0, 10000.0, causal, seed)


OFFSETS = [(0, 0), (64, 0), (40, 0), (500, 0), (0, 40), (0, 150), (0, 500), (1000, 1000), (77, 13)]
SHAPES = [(2, 100, 8, 2, 64), (1, 257, 4, 1, 128), (1, 130, 3, 3, 64), (2, 96, 8, 4, 128)]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}S{}H{}/{}d{}".format(*s))
def test_shard_offsets(shape, dtype):
    B, S, Hq, Hkv, d = shape
    w = w_of(B, S, Hq, Hkv, d, dtype, seed=S + d)
    q, k, v = make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for (qp, kp) in OFFSETS:
        for causal in (True, False):
            if not causal and (qp, kp) not in ((0, 0), (77, 13)):
                continue
            say(w, "q_pos0", qp, "k_pos0", kp, "causal", causal)
            out, lse = attn_fwd(qd, kd, vd, w.rope_theta, causal, q_pos0=qp, k_pos0=kp)
            torch.cuda.synchronize()
            ref_o, ref_l = attention(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                     w.rope_theta, causal, q_pos0=qp, k_pos0=kp)
            compare(dtype, out, lse, ref_o, ref_l, f"{w} offsets ({qp}, {kp}) causal {causal}")


@pytest.mark.parametrize("dtype,d,Hq,Hkv", [("bf16", 128, 8, 2), ("bf16", 64, 8, 8), ("fp32", 64, 4, 1)])
def test_ring_composition(dtype, d, Hq, Hkv):
    """Causal attention over S = 4 shards of n: each query shard merged over every key shard at
    its offset (later shards contribute empty rows), against the unsharded oracle."""
    n, parts = 256 if dtype == "bf16" else 64, 4
    S = n * parts
    w = w_of(1, S, Hq, Hkv, d, dtype, seed=d + Hkv)
    q, k, v = make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ref_o, ref_l = attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.rope_theta, True)
    for s in range(parts):
        say(w, "query shard", s)
        qs = qd[:, s * n:(s + 1) * n].contiguous()
        acc_o, acc_l = None, None
        for t in range(parts):
            ks, vs = kd[:, t * n:(t + 1) * n].contiguous(), vd[:, t * n:(t + 1) * n].contiguous()
            o, l = attn_fwd(qs, ks, vs, w.rope_theta, True, q_pos0=s * n, k_pos0=t * n)
            if acc_o is None:
                acc_o, acc_l = o, l
            else:
                attn_merge(acc_o, acc_l, o, l, out=acc_o, lse=acc_l)  # in place
        torch.cuda.synchronize()
        compare(dtype, acc_o, acc_l, ref_o[:, s * n:(s + 1) * n], ref_l[:, :, s * n:(s + 1) * n],
                f"{w} ring shard {s}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_merge_kernel(dtype, d):
    g = torch.Generator().manual_seed(d)
    B, S, H = 2, 77, 5
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o1 = torch.randn((B, S, H, d), generator=g).to(tdt)
    o2 = torch.randn((B, S, H, d), generator=g).to(tdt)
    l1 = torch.randn((B, H, S), generator=g) * 4.0
    l2 = torch.randn((B, H, S), generator=g) * 4.0 + 1.0
    l1[0, 1, :10] = -float("inf")  # part 1 empty
    l2[1, 2, 5:20] = -float("inf")  # part 2 empty
    l1[1, 0, 30:40] = -float("inf")
    l2[1, 0, 30:40] = -float("inf")  # both empty
    o1[0, :10, 1] = 0
    o2[1, 5:20, 2] = 0
    o1[1, 30:40, 0] = 0
    o2[1, 30:40, 0] = 0
    ref_o, ref_l = merge(o1.double().numpy(), l1.double().numpy(), o2.double().numpy(), l2.double().numpy())
    say("merge", dtype, d)
    out, lse = attn_merge(o1.cuda(), l1.cuda(), o2.cuda(), l2.cuda())
    torch.cuda.synchronize()
    compare(dtype, out, lse, ref_o, ref_l, f"merge {dtype} d{d}")
    # in place into the first part gives the same bits
    a, al = o1.cuda(), l1.cuda()
    attn_merge(a, al, o2.cuda(), l2.cuda(), out=a, lse=al)
    torch.cuda.synchronize()
    assert torch.equal(a, out) and torch.equal(al, lse)
