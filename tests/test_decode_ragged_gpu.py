"""GPU parity of the ragged-batch decode step (attn_decode_ragged), through the C ABI.

Each batch row b has its own position q_pos[b] (a device array): its query, placed at row
q_pos[b], attends to its cached keys 0 .. q_pos[b], i.e. row q_pos[b] of causal attention for
that batch row, so the oracle is attention(..., rows=[q_pos[b]]) on batch row b alone.  The
cache rows past a row's position hold NaN (prepared from NaN keys and values), so a read of
any key a row must not see would show.  Tolerance as for the bf16 forward: 2e-2 on out and lse.
"""

import numpy as np
import pytest
import torch

from oracle import attention
from transformer_causal_attention_amd import _lib, attn_decode, kv_prepare, new_kv_cache
from transformer_causal_attention_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(*a):
    print("[gpu-case]", *a, flush=True)


CASES = [
    # B, S_cap, Hq, Hkv, d, theta, positions, max_pos (None: S_cap - 1)
    (4, 2048, 32, 8, 128, 500000.0, [0, 63, 1500, 2047], None),
    (8, 1024, 8, 1, 64, 10000.0, [5, 1023, 64, 65, 0, 700, 31, 32], 1023),
    (3, 300, 8, 2, 128, 10000.0, [299, 1, 150], 299),
    (3, 1500, 48, 1, 256, 10000.0, [1499, 10, 777], None),
    (5, 512, 16, 4, 128, 10000.0, [100, 100, 3, 256, 200], 256),  # a tight bound
]


def build(case, seed=5):
    B, S, Hq, Hkv, d, theta, pos, _ = case
    w = Workload("ragged", B, S, Hq, Hkv, d, "bf16", 1.0, theta, True, seed + S)
    q, k, v = make_inputs(w)
    # keys and values past each row's position become NaN: the decode must never read them
    for b, p_ in enumerate(pos):
        k[b, p_ + 1:] = float("nan")
        v[b, p_ + 1:] = float("nan")
    return w, q, k, v


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}S{}H{}/{}d{}".format(*c[:5]))
def test_ragged_decode(case):
    B, S, Hq, Hkv, d, theta, pos, max_pos = case
    w, q, k, v = build(case)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cache = new_kv_cache(B, S, Hkv, d, "cuda")
    kv_prepare(kd, vd, theta, 0, S, cache)
    qrow = torch.stack([qd[b, p_] for b, p_ in enumerate(pos)]).contiguous()  # (B, Hq, d)
    qpos = torch.tensor(pos, dtype=torch.int32, device="cuda")
    say(case)
    out, lse = attn_decode(qrow, cache, S, Hkv, theta, qpos, max_pos=max_pos)
    torch.cuda.synchronize()
    o = out.float().cpu().double().numpy()
    l = lse.cpu().double().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    for b, p_ in enumerate(pos):
        # row b alone: keys up to p_ only (the oracle never sees the NaN rows after p_)
        n = p_ + 1
        ref_o, ref_l = attention(q[b:b + 1, :n].double().numpy(), k[b:b + 1, :n].double().numpy(),
                                 v[b:b + 1, :n].double().numpy(), theta, True, rows=[p_])
        eo = np.abs(o[b] - ref_o[0, 0]).max()
        el = np.abs(l[b] - ref_l[0, :, 0]).max()
        say(f"row {b} q_pos {p_}: out err {eo:.3e}, lse err {el:.3e}")
        assert eo <= TOL and el <= TOL


def test_ragged_equals_uniform_rows():
    # every row at the same position: the ragged call computes the uniform call's rows
    case = (3, 700, 8, 2, 128, 10000.0, [500, 500, 500], 500)
    B, S, Hq, Hkv, d, theta, pos, max_pos = case
    w, q, k, v = build(case)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cache = new_kv_cache(B, S, Hkv, d, "cuda")
    kv_prepare(kd, vd, theta, 0, S, cache)
    qrow = qd[:, 500].contiguous()
    o_u, l_u = attn_decode(qrow, cache, S, Hkv, theta, 500)
    o_r, l_r = attn_decode(qrow, cache, S, Hkv, theta, torch.tensor(pos, dtype=torch.int32, device="cuda"),
                           max_pos=max_pos)
    torch.cuda.synchronize()
    assert torch.equal(o_u, o_r) and torch.equal(l_u, l_r)


def test_ragged_position_beyond_bound_gives_nan_for_that_row_only():
    case = (3, 300, 8, 2, 128, 10000.0, [100, 250, 7], 200)  # row 1 exceeds max_pos
    B, S, Hq, Hkv, d, theta, pos, max_pos = case
    w, q, k, v = build(case)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cache = new_kv_cache(B, S, Hkv, d, "cuda")
    kv_prepare(kd, vd, theta, 0, S, cache)
    qrow = torch.stack([qd[b, p_] for b, p_ in enumerate(pos)]).contiguous()
    out, lse = attn_decode(qrow, cache, S, Hkv, theta, torch.tensor(pos, dtype=torch.int32, device="cuda"),
                           max_pos=max_pos)
    torch.cuda.synchronize()
    assert torch.isnan(out[1].float()).all() and torch.isnan(lse[1]).all()
    assert torch.isfinite(out[0].float()).all() and torch.isfinite(out[2].float()).all()
    assert torch.isfinite(lse[0]).all() and torch.isfinite(lse[2]).all()


def test_ragged_host_checks():
    q = torch.empty((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    cache = new_kv_cache(2, 256, 2, 128, "cuda")
    with pytest.raises(_lib.AttnError) as e:
        attn_decode(q, cache, 256, 2, 1e4, torch.zeros(2, dtype=torch.int32, device="cuda"), max_pos=256)
    assert e.value.code == _lib.ATTN_EINVAL
    with pytest.raises(ValueError):
        attn_decode(q, cache, 256, 2, 1e4, torch.zeros(3, dtype=torch.int32, device="cuda"))
