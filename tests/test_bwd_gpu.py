"""GPU parity of the backward pass (attn_bwd) against the float64 oracle's attention_backward.

The GPU forward supplies out and lse (as in training); the oracle recomputes everything from
q, k, v and dout in float64.  Tolerance, derived from the arithmetic: the kernels round the
rotated q and k, v, dout, P and dS to bf16 (relative error up to 2^-9 each) and accumulate in
fp32, so each gradient element carries a relative error of a few 2^-9 of the magnitude of its
terms; checked as max |err| <= 2e-2 * max(1, max |ref|) per tensor, and Frobenius error
<= 1e-2 * max(1, ||ref||) (a causal single row has dq = 0 exactly, so the floor of 1).
"""

import numpy as np
import pytest
import torch

from oracle import attention_backward
from transformer_causal_attention_amd import attn_bwd, attn_fwd
from transformer_causal_attention_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-case]", *a, flush=True)


def w_of(B, S, Hq, Hkv, d, causal, theta=10000.0, sigma=1.0, seed=9):
    return Workload("bwd", B, S, Hq, Hkv, d, "bf16", sigma, theta, causal, seed)


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


def run_case(w, q, k, v, do):
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = attn_fwd(qd, kd, vd, w.rope_theta, w.causal)
    dq, dk, dv = attn_bwd(qd, kd, vd, out, lse, dod, w.rope_theta, w.causal)
    torch.cuda.synchronize()
    return dq, dk, dv


SHAPES = [
    (1, 64, 4, 1, 64, True),     # MQA, one pair of blocks
    (2, 100, 8, 2, 128, True),   # GQA, ragged
    (1, 130, 3, 3, 64, False),   # MHA, ragged, full
    (1, 257, 8, 1, 128, True),   # 8 heads per K/V head: 4 waves, 2 heads each; odd block count
    (2, 96, 16, 2, 64, True),    # 8 heads per K/V head
    (1, 200, 6, 2, 128, False),  # 3 heads per K/V head: 3 waves
    (1, 33, 2, 1, 128, True),    # two blocks, second holds one row
    (3, 1, 4, 2, 64, True),      # single row
    (1, 100, 8, 1, 256, True),   # head_dim 256 (PaLM-540B's), multi-query, ragged
    (2, 70, 4, 2, 256, False),   # head_dim 256, full attention
    (1, 33, 2, 2, 256, True),    # head_dim 256, two blocks, second holds one row
    (1, 64, 48, 1, 256, True),   # PaLM-540B heads: 12 passes of 4 heads spread over 12 head splits
    (1, 80, 12, 1, 128, False),  # 3 passes over 3 head splits, full attention
    (1, 150, 2, 2, 128, True),   # MHA at head_dim 128: single-block work items for every kernel
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}S{}H{}/{}d{}{}".format(*s[:5], "c" if s[5] else "f"))
def test_bwd_parity(shape):
    B, S, Hq, Hkv, d, causal = shape
    w = w_of(B, S, Hq, Hkv, d, causal, seed=S + d + Hq)
    q, k, v = make_inputs(w)
    do = dout_of(w)
    say(w)
    dq, dk, dv = run_case(w, q, k, v, do)
    rq, rk, rv = attention_backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(),
                                    w.rope_theta, causal)
    check("dq", dq, rq, str(w))
    check("dk", dk, rk, str(w))
    check("dv", dv, rv, str(w))


def _random_shapes(n=12, seed=2024):
    """Seeded irregular shapes: group sizes 1-8 (MHA, GQA, MQA), head_dim 64 or 128, ragged
    lengths, causal or not; each picks its own launch forms (one launch or several, one pass or
    two at head_dim 64, head splits or none)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hkv = int(rng.choice([1, 2, 3, 4]))
        g = int(rng.choice([1, 2, 3, 4, 6, 8]))
        out.append((int(rng.integers(1, 4)), int(rng.integers(1, 330)), hkv * g, hkv, int(rng.choice([64, 128])),
                    bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("shape", _random_shapes(), ids=lambda s: "B{}S{}H{}/{}d{}{}".format(*s[:5], "c" if s[5] else "f"))
def test_bwd_parity_random_shapes(shape):
    B, S, Hq, Hkv, d, causal = shape
    w = w_of(B, S, Hq, Hkv, d, causal, seed=S * 7 + Hq + d)
    q, k, v = make_inputs(w)
    do = dout_of(w)
    say(w)
    dq, dk, dv = run_case(w, q, k, v, do)
    rq, rk, rv = attention_backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(),
                                    w.rope_theta, causal)
    check("dq", dq, rq, str(w))
    check("dk", dk, rk, str(w))
    check("dv", dv, rv, str(w))


def test_bwd_llama3_full_size_one_group():
    """Llama-3-8B shape (B1 S2048 Hq32 Hkv8 d128, rope_theta 5e5) in the benchmark's launch
    configuration; the oracle evaluates K/V group 3 (query heads 12..15), whose gradients do
    not depend on the other groups."""
    w = Workload("llama3_8b", 1, 2048, 32, 8, 128, "bf16", 1.0, 500000.0, True, 2)
    q, k, v = make_inputs(w)
    do = dout_of(w)
    say(w)
    dq, dk, dv = run_case(w, q, k, v, do)
    g = 3
    hs = slice(4 * g, 4 * g + 4)
    rq, rk, rv = attention_backward(q[:, :, hs].double().numpy(), k[:, :, g:g + 1].double().numpy(),
                                    v[:, :, g:g + 1].double().numpy(), do[:, :, hs].double().numpy(), w.rope_theta, True)
    check("dq", dq[:, :, hs], rq, "llama3 group 3")
    check("dk", dk[:, :, g:g + 1], rk, "llama3 group 3")
    check("dv", dv[:, :, g:g + 1], rv, "llama3 group 3")


@pytest.mark.parametrize("name,heads", [("palm_mqa", slice(0, 8)), ("smollm_mha", slice(5, 7))])
def test_bwd_full_size_one_batch_row(name, heads):
    """PaLM MQA (B8 S1024 Hq8 Hkv1 d64) and SmolLM MHA (B4 S1024 Hq32 Hkv32 d64) backward in the
    benchmark's launch configuration; the oracle evaluates batch row 1 (rows are independent),
    for SmolLM MHA only query heads 5 and 6 with their own K/V heads (heads are independent)."""
    from transformer_causal_attention_amd.workloads import WORKLOADS
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    do = dout_of(w)
    say(w)
    dq, dk, dv = run_case(w, q, k, v, do)
    bsl = slice(1, 2)
    kv = heads if w.Hkv == w.Hq else slice(0, w.Hkv)
    rq, rk, rv = attention_backward(q[bsl, :, heads].double().numpy(), k[bsl, :, kv].double().numpy(),
                                    v[bsl, :, kv].double().numpy(), do[bsl, :, heads].double().numpy(),
                                    w.rope_theta, w.causal)
    check("dq", dq[bsl, :, heads], rq, f"{name} row 1")
    check("dk", dk[bsl, :, kv], rk, f"{name} row 1")
    check("dv", dv[bsl, :, kv], rv, f"{name} row 1")


def test_bwd_deterministic():
    w = w_of(2, 150, 8, 2, 128, True, seed=77)
    q, k, v = make_inputs(w)
    do = dout_of(w)
    a = run_case(w, q, k, v, do)
    for _ in range(2):
        b = run_case(w, q, k, v, do)
        for x, y in zip(a, b):
            assert torch.equal(x, y)


@pytest.mark.parametrize("shape", [(2, 300, 8, 2, 128, True), (1, 200, 4, 4, 64, True), (2, 170, 16, 2, 64, False),
                                   (1, 96, 48, 1, 256, True)],
                         ids=lambda s: "B{}S{}H{}/{}d{}{}".format(*s[:5], "c" if s[5] else "f"))
def test_bwd_work_items_agree(shape, monkeypatch):
    """Block pairs and single blocks (heaviest first) are two orders of the same work: every
    block's sums run in the same order, so both give the same bits (ATTN_BWD_ITEMS forces one
    kind for every kernel, ATTN_BWD_KV=waves picks the dk/dv kernels that take such items;
    head_dim 256 always runs single blocks)."""
    B, S, Hq, Hkv, d, causal = shape
    w = w_of(B, S, Hq, Hkv, d, causal, seed=S + Hq)
    q, k, v = make_inputs(w)
    do = dout_of(w)
    say(w)
    monkeypatch.setenv("ATTN_BWD_KV", "waves")
    res = {}
    for items in ("pairs", "single"):
        monkeypatch.setenv("ATTN_BWD_ITEMS", items)
        res[items] = run_case(w, q, k, v, do)
    for name, a, b in zip(("dq", "dk", "dv"), res["pairs"], res["single"]):
        assert torch.equal(a, b), f"{w}: {name} differs between pairs and single blocks"


@pytest.mark.parametrize("shape", [(2, 300, 8, 2, 128, True), (1, 200, 4, 4, 64, True), (2, 170, 16, 2, 64, False),
                                   (1, 150, 2, 2, 128, True), (1, 257, 8, 1, 128, True), (2, 96, 16, 2, 64, True)],
                         ids=lambda s: "B{}S{}H{}/{}d{}{}".format(*s[:5], "c" if s[5] else "f"))
def test_bwd_one_launch_agrees(shape, monkeypatch):
    """dk, dv and (with four or more heads per K/V head) dq work items in one launch
    (interleaved, heaviest first), dk and dv in one and dq in another, or a launch each
    (ATTN_BWD_KVLAUNCH, ATTN_BWD_DQLAUNCH): every item computes the same sums, so the bits
    agree."""
    B, S, Hq, Hkv, d, causal = shape
    w = w_of(B, S, Hq, Hkv, d, causal, seed=S + Hq + 4)
    q, k, v = make_inputs(w)
    do = dout_of(w)
    say(w)
    res = {}
    for kind, kv, dq in (("split", "split", "split"), ("kv", "one", "split"), ("one", "one", "one")):
        monkeypatch.setenv("ATTN_BWD_KVLAUNCH", kv)
        monkeypatch.setenv("ATTN_BWD_DQLAUNCH", dq)
        res[kind] = run_case(w, q, k, v, do)
    for kind in ("kv", "one"):
        for name, a, b in zip(("dq", "dk", "dv"), res["split"], res[kind]):
            assert torch.equal(a, b), f"{w}: {name} differs between launches ({kind})"


@pytest.mark.parametrize("shape", [(1, 200, 4, 4, 64, True), (2, 170, 16, 2, 64, False), (2, 96, 16, 2, 64, True),
                                   (3, 1, 4, 2, 64, True), (1, 64, 4, 1, 64, True), (1, 520, 8, 1, 64, True)],
                         ids=lambda s: "B{}S{}H{}/{}d{}{}".format(*s[:5], "c" if s[5] else "f"))
def test_bwd_kv_fused_agrees(shape, monkeypatch):
    """At head_dim 64 one pass gives dk and dv together from the same probabilities and dS, summed
    in the same order as the two separate passes (ATTN_BWD_KVFUSE=off): the same bits."""
    B, S, Hq, Hkv, d, causal = shape
    w = w_of(B, S, Hq, Hkv, d, causal, seed=S + Hq + 6)
    q, k, v = make_inputs(w)
    do = dout_of(w)
    say(w)
    res = {}
    for kind in ("off", "on"):
        monkeypatch.setenv("ATTN_BWD_KVFUSE", kind)
        res[kind] = run_case(w, q, k, v, do)
    for name, a, b in zip(("dq", "dk", "dv"), res["off"], res["on"]):
        assert torch.equal(a, b), f"{w}: {name} differs between one pass and two"


@pytest.mark.parametrize("shape", [(2, 300, 8, 2, 128, True), (1, 200, 4, 4, 64, True), (2, 170, 16, 2, 64, False),
                                   (1, 150, 2, 2, 128, True)],
                         ids=lambda s: "B{}S{}H{}/{}d{}{}".format(*s[:5], "c" if s[5] else "f"))
def test_bwd_kv_kernels_agree(shape, monkeypatch):
    """dk and dv from the kernel that shares query blocks between four key blocks and from the
    one that gives each query head a wave: the same sums over the group's heads in another
    order, so they agree to a few bf16 roundings (ATTN_BWD_KV picks the kernel)."""
    B, S, Hq, Hkv, d, causal = shape
    w = w_of(B, S, Hq, Hkv, d, causal, seed=S + Hq + 3)
    q, k, v = make_inputs(w)
    do = dout_of(w)
    say(w)
    res = {}
    for kind in ("waves", "shared"):
        monkeypatch.setenv("ATTN_BWD_KV", kind)
        res[kind] = run_case(w, q, k, v, do)
    assert torch.equal(res["waves"][0], res["shared"][0]), f"{w}: dq depends on the dk/dv kernel"
    for name, a, b in zip(("dk", "dv"), res["waves"][1:], res["shared"][1:]):
        a, b = a.float(), b.float()
        err = (a - b).abs().max().item()
        scale = a.abs().max().item()
        assert err <= 2 ** -6 * scale, f"{w}: {name} max difference {err} (scale {scale})"


@pytest.mark.parametrize("shape", [(2, 300, 8, 2, 128, True), (1, 257, 8, 1, 128, True), (2, 96, 16, 2, 64, True),
                                   (1, 200, 6, 2, 128, False), (1, 200, 4, 4, 64, True), (2, 170, 4, 2, 128, False),
                                   (1, 150, 2, 2, 128, True), (1, 33, 2, 2, 64, True)],
                         ids=lambda s: "B{}S{}H{}/{}d{}{}".format(*s[:5], "c" if s[5] else "f"))
def test_bwd_dq_kernels_agree(shape, monkeypatch):
    """The dq kernel that shares each key block's tiles through LDS (between a group's heads, or
    between consecutive query blocks of one head) and the one that loads them per wave take the
    same operands in the same order: the same bits (ATTN_BWD_DQ picks the kernel)."""
    B, S, Hq, Hkv, d, causal = shape
    w = w_of(B, S, Hq, Hkv, d, causal, seed=S + Hq + 5)
    q, k, v = make_inputs(w)
    do = dout_of(w)
    say(w)
    res = {}
    for kind in ("regs", "shared"):
        monkeypatch.setenv("ATTN_BWD_DQ", kind)
        res[kind] = run_case(w, q, k, v, do)
    assert torch.equal(res["regs"][0], res["shared"][0]), f"{w}: dq differs between the two dq kernels"
