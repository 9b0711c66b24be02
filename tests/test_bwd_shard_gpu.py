"""GPU parity of one ring-attention backward step (attn_bwd_shard), through the C ABI.

Per step: the oracle's attention_backward_shard and the kernels receive the same q, k, v, dout
and the same out and lse (the float64 oracle forward's, rounded to bf16 and fp32), at offsets
that are and are not multiples of the 32-row blocks, causal and not, both rotary forms; rows
that see no key (lse -inf) must get no gradient.  End to end: a sequence of 3 blocks, forward
by shard calls merged on the GPU, then the 3 x 3 backward steps summed on the GPU, against the
oracle's backward of the whole sequence.  Tolerances as in the backward tests: max |err| <=
2e-2 * max(1, max |ref|) and Frobenius error <= 1e-2 * max(1, ||ref||) per tensor.
"""

import numpy as np
import pytest
import torch

from oracle import attention, attention_backward, attention_backward_shard
from transformer_causal_attention_amd import attn_bwd, attn_fwd, attn_merge
from transformer_causal_attention_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-case]", *a, flush=True)


def dout_of(w):
    g = torch.Generator().manual_seed(w.seed + 1000)
    return torch.randn((w.B, w.S, w.Hq, w.d), generator=g).to(torch.bfloat16)


def check(name, got, ref, what):
    g = got.float().cpu().double().numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
    err = np.abs(g - ref).max()
    scale = max(1.0, np.abs(ref).max())
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1.0)
    say(f"{what} {name}: max err {err:.3e} (scale {scale:.2f}), rel fro {rel:.3e}")
    assert err <= 2e-2 * scale and rel <= 1e-2, f"{what}: {name}"


STEPS = [
    # B, S, Hq, Hkv, d, causal, q_pos0, k_pos0, interleaved
    (1, 100, 8, 2, 128, True, 0, 0, False),
    (1, 100, 8, 2, 128, True, 64, 0, False),    # an earlier key block, block-aligned
    (2, 130, 4, 1, 64, True, 40, 0, False),     # earlier keys, offset not a multiple of 32
    (1, 96, 8, 2, 128, True, 77, 13, True),
    (1, 120, 6, 2, 64, True, 0, 40, False),     # a later key block: rows 0..39 see nothing
    (1, 90, 8, 1, 128, True, 13, 77, False),
    (1, 160, 8, 2, 128, True, 500, 0, False),   # every key visible to every row
    (1, 100, 8, 2, 64, False, 300, 7, True),    # full attention: offsets rotate only
    (1, 96, 4, 1, 256, True, 40, 0, False),     # head_dim 256, offset not a multiple of 32
    (1, 70, 4, 1, 256, True, 13, 77, True),     # head_dim 256, rows that see nothing
]


@pytest.mark.parametrize("case", STEPS, ids=lambda c: "B{}S{}H{}/{}d{}c{}q{}k{}i{}".format(*[int(x) for x in c]))
def test_backward_step_matches_oracle(case):
    B, S, Hq, Hkv, d, causal, qp, kp, il = case
    w = Workload("bwd_shard", B, S, Hq, Hkv, d, "bf16", 1.0, 5e5, causal, 17 + qp + kp)
    q, k, v = make_inputs(w)
    do = dout_of(w)
    qn, kn, vn, don = (t.double().numpy() for t in (q, k, v, do))
    # the same out (bf16) and lse (fp32) for both sides: this block's own forward
    o_ref, l_ref = attention(qn, kn, vn, w.rope_theta, causal, q_pos0=qp, k_pos0=kp, interleaved=il)
    out = torch.from_numpy(o_ref).to(torch.bfloat16)
    lse = torch.from_numpy(l_ref).to(torch.float32)
    refs = attention_backward_shard(qn, kn, vn, don, out.double().numpy(), lse.double().numpy(), w.rope_theta,
                                    causal, q_pos0=qp, k_pos0=kp, interleaved=il)
    say(case)
    grads = attn_bwd(q.cuda(), k.cuda(), v.cuda(), out.cuda(), lse.cuda(), do.cuda(), w.rope_theta, causal,
                     q_pos0=qp, k_pos0=kp, interleaved=il)
    torch.cuda.synchronize()
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        check(name, got, ref, str(case))
    if causal and kp > qp:
        # rows before the block's first key see nothing: exactly no gradient
        assert not grads[0][:, : kp - qp].float().any()


@pytest.mark.parametrize("d,il", [(128, False), (64, True)])
def test_ring_backward_end_to_end(d, il):
    n, parts = 96, 3
    w = Workload("ring_bwd", 1, n * parts, 8, 2, d, "bf16", 1.0, 5e5, True, 29)
    q, k, v = make_inputs(w)
    do = dout_of(w)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    sl = [slice(a * n, (a + 1) * n) for a in range(parts)]
    blk = lambda t, a: t[:, sl[a]].contiguous()  # noqa: E731
    # forward of each query block over the key blocks it sees, merged on the GPU
    outs, lses = [], []
    for a in range(parts):
        o, l = None, None
        for c in range(a + 1):
            ot, lt = attn_fwd(blk(qd, a), blk(kd, c), blk(vd, c), w.rope_theta, True, q_pos0=a * n, k_pos0=c * n,
                              interleaved=il)
            o, l = (ot, lt) if o is None else attn_merge(o, l, ot, lt)
        outs.append(o)
        lses.append(l)
    dq = torch.zeros(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.zeros(k.shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros(v.shape, dtype=torch.float32, device="cuda")
    for a in range(parts):
        for c in range(a + 1):
            say(f"ring backward step q block {a}, k block {c}")
            gq, gk, gv = attn_bwd(blk(qd, a), blk(kd, c), blk(vd, c), outs[a], lses[a], blk(dod, a), w.rope_theta,
                                  True, q_pos0=a * n, k_pos0=c * n, interleaved=il)
            dq[:, sl[a]] += gq.float()
            dk[:, sl[c]] += gk.float()
            dv[:, sl[c]] += gv.float()
    torch.cuda.synchronize()
    refs = attention_backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(),
                              w.rope_theta, True, interleaved=il)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        check(name, got, ref, f"ring d={d}")
