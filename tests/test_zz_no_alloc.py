"""attn_fwd_noalloc (the library's fixed scratch as workspace, nothing allocated by the call)
against attn_fwd, through the C ABI: two calls in a row on one GPU, the second smaller, each
bit-identical to attn_fwd on the same inputs (same kernels, same arithmetic), plus the same
max-abs 2e-2 bar against the float64 oracle on sampled rows.  Calls too large for the scratch
are refused before any HIP call."""

import numpy as np
import pytest
import torch

from oracle import attention
from transformer_causal_attention_amd import _lib, attn_fwd, attn_fwd_noalloc
from transformer_causal_attention_amd.workloads import WORKLOADS, Workload, make_inputs

TOL = 2e-2


def say(*a):
    print("[gpu-case]", *a, flush=True)


def one(w, rows):
    q, k, v = make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device="cuda")
    say("noalloc", w)
    attn_fwd_noalloc(qd, kd, vd, w.rope_theta, w.causal, out, lse)
    torch.cuda.synchronize()
    say("attn_fwd", w)
    ref_o, ref_l = attn_fwd(qd, kd, vd, w.rope_theta, w.causal)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), "attn_fwd_noalloc differs from attn_fwd"
    o_or, l_or = attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.rope_theta, w.causal, rows)
    eo = float(np.abs(out.float().cpu().double().numpy()[:, rows] - o_or).max())
    el = float(np.abs(lse.cpu().double().numpy()[:, :, rows] - l_or).max())
    say(f"{w.name}: out err {eo:.3e}, lse err {el:.3e}")
    assert eo <= TOL and el <= TOL


@pytest.mark.gpu
def test_noalloc_two_calls_match_attn_fwd():
    big = WORKLOADS["llama3_8b"]
    one(big, np.array([0, 1, 63, 64, 1000, 2046, 2047]))
    smaller = Workload("smaller", 2, 300, 8, 2, 128, "bf16", 1.0, 10000.0, True, 21)
    one(smaller, np.arange(0, 300, 13))


@pytest.mark.gpu
def test_noalloc_refuses_calls_beyond_the_scratch():
    w = WORKLOADS["long_shard"]  # 128 MiB of prepared tiles > 64 MiB of scratch
    q = torch.empty((w.B, w.S, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((w.B, w.S, w.Hkv, w.d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device="cuda")
    with pytest.raises(_lib.AttnError) as e:
        attn_fwd_noalloc(q, k, k, w.rope_theta, w.causal, out, lse)
    assert e.value.code == _lib.ATTN_ESCRATCH
