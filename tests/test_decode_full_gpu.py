"""GPU parity of the decode step at the sizes its benchmark times, on sampled batch rows.

The whole batch is prepared and decoded in one call each (the launch configuration of the
timed step: the split count and grid follow from B, Hq, Hkv, head_dim and q_pos), and the
first and last batch rows are checked against the float64 oracle, which evaluates only the
decode row (a broadcast query view: the oracle copies the rows it is asked for).  Tolerance
as for the other bf16 tests: max-abs 2e-2 on out and lse.
"""

import numpy as np
import pytest
import torch

from oracle import attention
from transformer_causal_attention_amd import attn_decode, kv_prepare, new_kv_cache

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print("[gpu-case]", *a, flush=True)


def inputs(B, S, Hq, Hkv, d, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn((B, S, Hkv, d), generator=g).to(torch.bfloat16)
    v = torch.randn((B, S, Hkv, d), generator=g).to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=g).to(torch.bfloat16)
    return q, k, v


# (B, S_cap, Hq, Hkv, d, rope_theta): Llama-3-8B heads over a full 32K cache at batch 8, and
# PaLM-540B heads (48 on one K/V head, head_dim 256) over 2048 keys at batch 64
CASES = [
    (8, 32768, 32, 8, 128, 500000.0),
    (64, 2048, 48, 1, 256, 10000.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}S{}H{}/{}d{}".format(*c[:5]))
def test_decode_full_size_sampled_rows(case):
    B, S, Hq, Hkv, d, theta = case
    q, k, v = inputs(B, S, Hq, Hkv, d, seed=S + d)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cache = new_kv_cache(B, S, Hkv, d, "cuda")
    kv_prepare(kd, vd, theta, 0, S, cache)
    sample = [0, B - 1]
    for pos in (S - 1, S // 2 + 5):
        say(case, "q_pos", pos)
        out, lse = attn_decode(qd, cache, S, Hkv, theta, pos)
        torch.cuda.synchronize()
        o = out.float().cpu().double().numpy()[sample]
        l = lse.cpu().double().numpy()[sample]
        qs = q[sample].double().numpy()
        qv = np.broadcast_to(qs[:, None], (len(sample), S, Hq, d))
        ref_o, ref_l = attention(qv, k[sample].double().numpy(), v[sample].double().numpy(), theta, True,
                                 rows=[pos])
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
        eo = np.abs(o - ref_o[:, 0]).max()
        el = np.abs(l - ref_l[:, :, 0]).max()
        say(f"B{B} S{S} d{d} q_pos {pos}: out err {eo:.3e}, lse err {el:.3e}")
        assert eo <= TOL and el <= TOL
