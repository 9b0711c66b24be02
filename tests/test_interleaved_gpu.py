"""GPU parity of the adjacent-pair (interleaved) rotary form against the float64 oracle.

Every entry point that rotates q or k takes rope_style; with ATTN_ROPE_INTERLEAVED dims
(2i, 2i+1) turn together by frequency i (the llama3-from-scratch page's complex-number
rotation) instead of (i, i + d/2).  The oracle's attention(..., interleaved=True) and
attention_backward(..., interleaved=True) are the references; tolerances are those of the
half-split tests (2e-2 for bf16 out/lse, 1e-4 for float32, the gradient bound of the backward
tests).  One case also checks that the flag changes the result, so a path that ignored it
could not pass.
"""

import numpy as np
import pytest
import torch

from oracle import attention, attention_backward
from transformer_causal_attention_amd import attn_bwd, attn_decode, attn_fwd, kv_prepare, new_kv_cache
from transformer_causal_attention_amd.workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def say(*a):
    print("[gpu-case]", *a, flush=True)


def np64(t):
    return t.double().numpy()


def compare(w, out, lse, ref_out, ref_lse, what):
    o = out.float().cpu().double().numpy()
    l = lse.cpu().double().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), f"{what}: non-finite output"
    eo, el = np.abs(o - ref_out).max(), np.abs(l - ref_lse).max()
    say(f"{what}: out err {eo:.3e}, lse err {el:.3e}")
    assert eo <= TOL[w.dtype] and el <= TOL[w.dtype], what


def w_of(B, S, Hq, Hkv, d, dtype, causal=True, theta=10000.0, seed=11):
    return Workload("il", B, S, Hq, Hkv, d, dtype, 1.0, theta, causal, seed)


FWD = []
for d in (64, 128):
    for (B, S, Hq, Hkv, causal) in ((1, 100, 4, 1, True), (2, 257, 8, 2, True), (1, 130, 3, 3, False),
                                    (1, 64, 8, 1, True), (2, 7, 2, 2, True)):
        FWD.append(w_of(B, S, Hq, Hkv, d, "bf16", causal, seed=S + d))
    FWD.append(w_of(1, 100, 4, 1, d, "fp32", True, seed=d + 1))
    FWD.append(w_of(2, 65, 6, 2, d, "fp32", False, seed=d + 2))


@pytest.mark.parametrize("w", FWD, ids=lambda w: f"{w.dtype}-B{w.B}S{w.S}H{w.Hq}/{w.Hkv}d{w.d}{'c' if w.causal else 'f'}")
def test_forward(w):
    q, k, v = make_inputs(w)
    say(w)
    out, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), w.rope_theta, w.causal, interleaved=True)
    torch.cuda.synchronize()
    ref_o, ref_l = attention(np64(q), np64(k), np64(v), w.rope_theta, w.causal, interleaved=True)
    compare(w, out, lse, ref_o, ref_l, f"{w} interleaved")


def test_forward_llama3_full_size_and_flag_matters():
    w = WORKLOADS["llama3_8b"]
    q, k, v = make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    say(w, "interleaved")
    out, lse = attn_fwd(qd, kd, vd, w.rope_theta, w.causal, interleaved=True)
    half, _ = attn_fwd(qd, kd, vd, w.rope_theta, w.causal)
    torch.cuda.synchronize()
    ref_o, ref_l = attention(np64(q), np64(k), np64(v), w.rope_theta, w.causal, interleaved=True)
    compare(w, out, lse, ref_o, ref_l, f"{w} interleaved")
    diff = (out.float() - half.float()).abs().max().item()
    say(f"max |interleaved - half-split| = {diff:.3e}")
    assert diff > 0.1, "the rotary style flag did not change the result"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_shard_offsets(dtype):
    w = w_of(2, 96, 8, 2, 128, dtype, seed=21)
    q, k, v = make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for (qp, kp) in ((64, 0), (0, 40), (77, 13), (1000, 1000)):
        say(w, "q_pos0", qp, "k_pos0", kp)
        out, lse = attn_fwd(qd, kd, vd, w.rope_theta, True, q_pos0=qp, k_pos0=kp, interleaved=True)
        torch.cuda.synchronize()
        ref_o, ref_l = attention(np64(q), np64(k), np64(v), w.rope_theta, True, q_pos0=qp, k_pos0=kp,
                                 interleaved=True)
        o, l = out.float().cpu().double().numpy(), lse.cpu().double().numpy()
        seen = np.isfinite(ref_l)
        assert np.all(l[~seen] == -np.inf) and np.all(np.isfinite(o)), "empty rows"
        eo = np.abs(o - ref_o).max()
        el = np.abs(l[seen] - ref_l[seen]).max() if np.any(seen) else 0.0
        say(f"offsets ({qp}, {kp}): out err {eo:.3e}, lse err {el:.3e}")
        assert eo <= TOL[dtype] and el <= TOL[dtype]


@pytest.mark.parametrize("shape", [(1, 300, 8, 2, 128), (2, 130, 8, 1, 64), (1, 260, 48, 1, 256)], ids=lambda s: "B{}S{}H{}/{}d{}".format(*s))
def test_decode(shape):
    B, S, Hq, Hkv, d = shape
    w = w_of(B, S, Hq, Hkv, d, "bf16", seed=S)
    q, k, v = make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    cache = new_kv_cache(B, S, Hkv, d, "cuda")
    kv_prepare(kd, vd, w.rope_theta, 0, S, cache, interleaved=True)
    for pos in (0, 63, 64, S // 2, S - 1):
        say(w, "q_pos", pos)
        out, lse = attn_decode(qd[:, pos].contiguous(), cache, S, Hkv, w.rope_theta, pos, interleaved=True)
        torch.cuda.synchronize()
        ref_o, ref_l = attention(np64(q), np64(k), np64(v), w.rope_theta, True, rows=[pos], interleaved=True)
        eo = np.abs(out.float().cpu().double().numpy() - ref_o[:, 0]).max()
        el = np.abs(lse.cpu().double().numpy() - ref_l[:, :, 0]).max()
        say(f"q_pos {pos}: out err {eo:.3e}, lse err {el:.3e}")
        assert eo <= TOL["bf16"] and el <= TOL["bf16"]


@pytest.mark.parametrize("shape", [(2, 100, 8, 2, 128, True), (1, 130, 3, 3, 64, False), (1, 64, 4, 1, 64, True)],
                         ids=lambda s: "B{}S{}H{}/{}d{}{}".format(*s[:5], "c" if s[5] else "f"))
def test_backward(shape):
    B, S, Hq, Hkv, d, causal = shape
    w = w_of(B, S, Hq, Hkv, d, "bf16", causal, seed=S + Hq)
    q, k, v = make_inputs(w)
    g = torch.Generator().manual_seed(w.seed + 1000)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    say(w, "backward")
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = attn_fwd(qd, kd, vd, w.rope_theta, causal, interleaved=True)
    grads = attn_bwd(qd, kd, vd, out, lse, dod, w.rope_theta, causal, interleaved=True)
    torch.cuda.synchronize()
    refs = attention_backward(np64(q), np64(k), np64(v), np64(do), w.rope_theta, causal, interleaved=True)
    for name, got, ref in zip(("dq", "dk", "dv"), grads, refs):
        gv = got.float().cpu().double().numpy()
        err = np.abs(gv - ref).max()
        scale = max(1.0, np.abs(ref).max())
        rel = np.linalg.norm(gv - ref) / max(np.linalg.norm(ref), 1.0)
        say(f"{name}: max err {err:.3e} (scale {scale:.2f}), rel fro {rel:.3e}")
        assert np.all(np.isfinite(gv)) and err <= 2e-2 * scale and rel <= 1e-2, name
