"""GPU parity: the HIP path (through the C ABI) against the float64 oracle, element by element.

Tolerances: max-abs error of out and of lse <= 2e-2 for bf16 inputs, <= 1e-4 for float32
inputs, on identical seeded inputs.  Small shapes span several tiles with ragged tails; the
five workload shapes run at full size (the 32K-token shard is compared on sampled rows the
oracle evaluates one by one, in the same launch configuration the benchmark times).
"""

import numpy as np
import pytest
import torch

from oracle import attention
from transformer_causal_attention_amd import AttnError, Event, attn_fwd, attn_fwd_into
from transformer_causal_attention_amd.workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def say(*a):
    print("[gpu-case]", *a, flush=True)


def gpu_run(w, q, k, v, **kw):
    say(w)
    out, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), w.rope_theta, w.causal, **kw)
    torch.cuda.synchronize()
    return out, lse


def oracle_run(w, q, k, v, rows=None):
    return attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), w.rope_theta, w.causal, rows)


def compare(w, out, lse, ref_out, ref_lse, rows=None):
    o = out.float().cpu().double().numpy()
    l = lse.cpu().double().numpy()
    if rows is not None:
        o = o[:, rows]
        l = l[:, :, rows]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), "non-finite output"
    eo = np.abs(o - ref_out)
    el = np.abs(l - ref_lse)
    tol = TOL[w.dtype]
    worst = np.unravel_index(np.argmax(eo), eo.shape)
    msg = f"{w}: out err {eo.max():.3e} at (b,row,h,c)={worst}, lse err {el.max():.3e}"
    say(msg)
    assert eo.max() <= tol, msg
    assert el.max() <= tol, msg


def small(name, B, S, Hq, Hkv, d, dtype, causal, theta=10000.0, sigma=1.0, seed=7):
    return Workload(name, B, S, Hq, Hkv, d, dtype, sigma, theta, causal, seed)


SMALL = []
for d in (64, 128):
    for (Hq, Hkv) in ((4, 1), (8, 2), (2, 2), (6, 2), (8, 1)):
        for S in (1, 7, 64, 100, 257):
            SMALL.append(small("s", 1 + (S % 2), S, Hq, Hkv, d, "bf16", True, seed=S + d))
for d in (64, 128):
    for (Hq, Hkv, S) in ((4, 1, 100), (8, 2, 257), (3, 3, 130), (8, 1, 65)):
        SMALL.append(small("nc", 2, S, Hq, Hkv, d, "bf16", False, theta=500000.0, seed=S))
        SMALL.append(small("f32", 1, S, Hq, Hkv, d, "fp32", True, seed=S + 1))
        SMALL.append(small("f32nc", 2, S, Hq, Hkv, d, "fp32", False, seed=S + 2))


@pytest.mark.parametrize("w", SMALL, ids=lambda w: f"{w.name}-B{w.B}S{w.S}H{w.Hq}/{w.Hkv}d{w.d}")
def test_small_shapes(w):
    q, k, v = make_inputs(w)
    out, lse = gpu_run(w, q, k, v)
    ref_out, ref_lse = oracle_run(w, q, k, v)
    compare(w, out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("name", ["tiny_mqa_fp32", "llama3_8b", "palm_mqa", "smollm_mha"])
def test_workload_full(name):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    out, lse = gpu_run(w, q, k, v)
    ref_out, ref_lse = oracle_run(w, q, k, v)
    compare(w, out, lse, ref_out, ref_lse)


def long_shard_rows(S, seed=5):
    # 32-row blocks: both blocks of three of the pairs (r, n-1-r) that one workgroup runs (the
    # first, the second and the middle pair), and six seeded random blocks
    n = S // 32
    fixed = [0, n - 1, 1, n - 2, n // 2 - 1, n // 2]
    rng = np.random.default_rng(seed)
    rest = sorted(rng.choice(np.setdiff1d(np.arange(n), fixed), size=6, replace=False).tolist())
    return np.concatenate([np.arange(32 * b, 32 * b + 32) for b in sorted(fixed + rest)])


def test_long_shard_sampled_rows():
    w = WORKLOADS["long_shard"]
    q, k, v = make_inputs(w)
    out, lse = gpu_run(w, q, k, v)
    rows = long_shard_rows(w.S)
    say(f"long shard: comparing {len(rows)} rows x {w.Hq} heads")
    ref_out, ref_lse = oracle_run(w, q, k, v, rows=rows)
    compare(w, out, lse, ref_out, ref_lse, rows=rows)
    # every row of every head is finite
    assert torch.isfinite(out).all().item() and torch.isfinite(lse).all().item()


def test_row0_is_exactly_v0():
    # Row 0 sees only key 0: weight exp2(0) = 1 and sum 1, so out_0 = v_0 bit for bit.
    w = small("row0", 2, 130, 8, 2, 128, "bf16", True)
    q, k, v = make_inputs(w)
    out, _ = gpu_run(w, q, k, v)
    o = out.cpu()
    for h in range(w.Hq):
        assert torch.equal(o[:, 0, h], v[:, 0, h // (w.Hq // w.Hkv)]), f"head {h}"


def test_zero_query_gives_running_mean():
    w = small("q0", 1, 200, 4, 1, 64, "bf16", True)
    q, k, v = make_inputs(w)
    q = torch.zeros_like(q)
    out, lse = gpu_run(w, q, k, v)
    vm = v[0, :, 0].double()
    mean = torch.cumsum(vm, 0) / torch.arange(1, w.S + 1, dtype=torch.float64)[:, None]
    for h in range(w.Hq):
        assert (out[0, :, h].cpu().double() - mean).abs().max().item() <= 2e-2
        assert (lse[0, h].cpu().double() - torch.log(torch.arange(1, w.S + 1, dtype=torch.float64))).abs().max().item() <= 2e-2


# Inputs with a wide score range, built in the lowest-frequency rotation pair (dimensions
# d/2 - 1 and d - 1): at rope_theta 5e5 it turns by under 1e-3 rad over a few hundred
# positions, so values placed there keep their size after rotation.  A kernel that takes
# probabilities against a running maximum must rescale when a later block scores far above
# the first one; these cases force that on every workgroup shape (1, 2 and 4 heads per
# K/V tile), causal and not, at both head sizes.
WIDE = [(d, Hq, Hkv, causal) for d in (64, 128) for (Hq, Hkv) in ((4, 1), (8, 2), (2, 2)) for causal in (True, False)]


def wide_ids(c):
    return f"d{c[0]}-H{c[1]}/{c[2]}-{'causal' if c[3] else 'full'}"


@pytest.mark.parametrize("depth", [55.0, 96.0])
@pytest.mark.parametrize("case", WIDE, ids=wide_ids)
def test_sunken_first_tile(case, depth):
    """Keys 0..63 score `depth` (natural units) below the later keys for rows >= 64.

    At depth 55 the later blocks' probability sums against the first block's maximum are
    about 2^79 (finite, above 2^64); at depth 96 they overflow float32.  Rows below 64 see
    only the first tile, with moderate scores.  Tolerances are the bf16 ones: the sunken keys
    carry weights of e^-55 or less, so their (larger) score rounding does not reach the result.
    """
    d, Hq, Hkv, causal = case
    w = small("sunken", 1, 300, Hq, Hkv, d, "bf16", causal, theta=500000.0, seed=int(depth) + d)
    q, k, v = (t.float() for t in make_inputs(w))
    c, c2 = d // 2 - 1, d - 1
    q, k = 0.5 * q, 0.5 * k
    k[:, :64] = 0.0
    k[:, :64, :, c] = -8.0
    k[:, 64:, :, c] = 0.0
    k[:, 64:, :, c2] = 0.0
    q[:, :64, :, c] = 0.5
    q[:, 64:, :, c] = depth * d ** 0.5 / 8.0
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    out, lse = gpu_run(w, q, k, v)
    ref_out, ref_lse = oracle_run(w, q, k, v)
    compare(w, out, lse, ref_out, ref_lse)


@pytest.mark.parametrize("case", WIDE, ids=wide_ids)
def test_staircase_scores(case):
    """Every 64-key tile scores about 68 (natural units) above the one before it.

    Each new tile's probabilities against the previous maximum sum past 2^97, so every tile is
    rescaled.  out keeps the bf16 tolerance.  For lse the scaled query is rounded to bf16
    (relative error up to 2^-9), which moves the top score of a row by up to 2^-9 * |s|;
    scores reach ~300 here, so lse is checked to 2e-2 + 2^-8 * max|s| per row.
    """
    d, Hq, Hkv, causal = case
    w = small("stairs", 1, 300, Hq, Hkv, d, "bf16", causal, theta=500000.0, seed=d + 3)
    q, k, v = (t.float() for t in make_inputs(w))
    c, c2 = d // 2 - 1, d - 1
    q, k = 0.25 * q, 0.25 * k
    q[..., c] = 68.0 * d ** 0.5 / 8.0
    q[..., c2] = 0.0
    k[..., c2] = 0.0
    k[..., c] = 8.0 * (torch.arange(w.S) // 64).float()[None, :, None]
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    out, lse = gpu_run(w, q, k, v)
    ref_out, ref_lse = oracle_run(w, q, k, v)
    o = out.float().cpu().double().numpy()
    assert np.all(np.isfinite(o))
    eo = np.abs(o - ref_out).max()
    # |s| of every row's top score, from the oracle's own lse (lse >= max score >= lse - ln S)
    lse_tol = 2e-2 + 2.0 ** -8 * (np.abs(ref_lse) + np.log(w.S))
    el = np.abs(lse.cpu().double().numpy() - ref_lse)
    say(f"staircase {w}: out err {eo:.3e}, lse err {el.max():.3e} (tol up to {lse_tol.max():.3e})")
    assert eo <= TOL["bf16"]
    assert np.all(el <= lse_tol)


def test_deterministic_and_overwrites_poisoned_outputs():
    w = small("det", 2, 300, 8, 2, 128, "bf16", True)
    q, k, v = (t.cuda() for t in make_inputs(w))
    say(w)
    out0, lse0 = attn_fwd(q, k, v, w.rope_theta, True)
    for _ in range(3):
        out = torch.full_like(out0, float("nan"))
        lse = torch.full_like(lse0, float("nan"))
        attn_fwd_into(q, k, v, w.rope_theta, True, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, out0) and torch.equal(lse, lse0)


# Many workgroups, several row-block pairs per (batch row, K/V head), every heads-per-group
# shape: a race between the waves of a workgroup shows up as runs that differ or overflow.
REPEAT = [small("rep", 4, 1024, Hq, Hkv, d, "bf16", True, sigma=0.5, seed=11)
          for d in (64, 128) for (Hq, Hkv) in ((16, 16), (16, 8), (32, 8))]


@pytest.mark.parametrize("w", REPEAT, ids=lambda w: f"B{w.B}S{w.S}H{w.Hq}/{w.Hkv}d{w.d}")
def test_repeated_runs_bit_identical(w):
    q, k, v = (t.cuda() for t in make_inputs(w))
    say(w)
    out0, lse0 = attn_fwd(q, k, v, w.rope_theta, True)
    torch.cuda.synchronize()
    assert torch.isfinite(out0).all() and torch.isfinite(lse0).all()
    # each output is a convex combination of value rows (bf16 rounding aside)
    assert out0.float().abs().max().item() <= 1.01 * v.float().abs().max().item()
    for _ in range(5):
        out, lse = attn_fwd(q, k, v, w.rope_theta, True)
        torch.cuda.synchronize()
        assert torch.equal(out, out0) and torch.equal(lse, lse0)


def test_canary_tails_untouched():
    for dtype in ("bf16", "fp32"):
        w = small("canary", 1, 77, 4, 2, 64, dtype, True)
        q, k, v = (t.cuda() for t in make_inputs(w))
        say(w)
        n_out = q.numel()
        big_out = torch.full((n_out + 4096,), 7.0, dtype=q.dtype, device="cuda")
        big_lse = torch.full((w.B * w.Hq * w.S + 1024,), 7.0, dtype=torch.float32, device="cuda")
        out = big_out[:n_out].view(q.shape)
        lse = big_lse[: w.B * w.Hq * w.S].view(w.B, w.Hq, w.S)
        ws = torch.full((1 << 20,), 0x5A, dtype=torch.uint8, device="cuda")
        attn_fwd_into(q, k, v, w.rope_theta, True, out, lse, workspace=ws if dtype == "bf16" else None)
        torch.cuda.synchronize()
        assert (big_out[n_out:] == 7.0).all().item()
        assert (big_lse[w.B * w.Hq * w.S:] == 7.0).all().item()


def test_side_stream_and_timed_events():
    w = WORKLOADS["palm_mqa"]
    q, k, v = (t.cuda() for t in make_inputs(w))
    say(w, "side stream")
    ref_out, ref_lse = attn_fwd(q, k, v, w.rope_theta, True)
    s = torch.cuda.Stream()
    e0, e1 = Event(), Event()
    with torch.cuda.stream(s):
        out, lse = attn_fwd(q, k, v, w.rope_theta, True, stream=s, events=(e0, e1))
    s.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    assert e0.elapsed_ms(e1) > 0.0


def test_errors_raise():
    q = torch.zeros((1, 8, 2, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(AttnError):
        attn_fwd(q, q[:, :, :1].contiguous(), q[:, :, :1].contiguous(), 10000.0, True)
    q = torch.zeros((1, 8, 3, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(AttnError):
        attn_fwd(q, kv, kv, 10000.0, True)
