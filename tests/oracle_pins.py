"""Pins that tie the float64 oracle to facts outside itself.

Each pin raises AssertionError on failure.  They are plain functions so that the mutation
test can run the whole set against deliberately broken copies of the oracle and show that
every plausible slip is caught by at least one of them.

What each pin rests on:
  * brute force      -- an independent pure-Python evaluation on tiny shapes (bruteforce.py);
  * softmax facts    -- rows of the weights sum to 1; weights of future keys are exactly 0;
  * closed forms     -- row 0 sees only key 0 (out = v_0, lse = q_0.k_0/sqrt(d) since the
                        rotation at position 0 is the identity); q = 0 gives uniform weights
                        (out_i = mean of v_0..v_i, lse_i = ln(i+1)); constant v gives that
                        constant; a strongly dominant diagonal gives out_i = v_i;
  * GQA              -- equals plain MHA on K/V heads repeated G times (contiguous groups);
  * rotation facts   -- norm preserved, dot products depend only on the position difference,
                        identity at position 0, d=2 is the textbook 2x2 rotation by p radians,
                        frequencies agree with the llama3 page's 1/theta**(arange(64)/64);
  * library routines -- torch's scaled_dot_product_attention (float64, CPU) on rotated q/k,
                        scipy's logsumexp for lse;
  * other page form  -- the llama3 page's adjacent-pair complex rotation equals the
                        half-split rotation after a fixed permutation of head_dim;
  * lse meaning      -- two disjoint key sets merged by logaddexp reproduce the full result;
  * golden fixtures  -- hand-derived closed-form cases in tests/golden/;
  * backward         -- central finite differences of the forward oracle (sum of dout * out)
                        on tiny shapes; the value gradient sums to the output gradient over
                        keys (softmax rows sum to 1); row 0 of dq is exactly 0 under the causal
                        mask (one visible key, so the softmax has nothing to trade off).
"""

import json
import math
import os

import numpy as np

import bruteforce
from oracle import attn_oracle as O

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------- brute force
BRUTE_CASES = [
    # (B, S, Hq, Hkv, d, causal, rope_theta)
    (1, 1, 1, 1, 2, True, 10000.0),
    (1, 5, 2, 1, 4, True, 10000.0),
    (2, 6, 4, 2, 8, True, 100.0),
    (1, 7, 3, 3, 4, False, 10000.0),
    (1, 8, 4, 1, 8, False, 500000.0),
    (1, 6, 4, 4, 2, True, 3.0),
    (1, 8, 2, 2, 6, True, 50.0),
]


def pin_bruteforce():
    rng = np.random.default_rng(11)
    for (B, S, Hq, Hkv, d, causal, theta) in BRUTE_CASES:
        q = _rand(rng, B, S, Hq, d, scale=0.7)
        k = _rand(rng, B, S, Hkv, d, scale=0.7)
        v = _rand(rng, B, S, Hkv, d)
        out_b, lse_b = bruteforce.brute_attention(q.tolist(), k.tolist(), v.tolist(), theta, causal)
        out_o, lse_o = O.attention(q, k, v, theta, causal=causal)
        case = f"brute force {(B, S, Hq, Hkv, d, causal, theta)}"
        _close(out_o, out_b, 1e-12, case + " out")
        _close(lse_o, lse_b, 1e-12, case + " lse")


# ---------------------------------------------------------------- softmax facts
def _rotated(rng, B=1, S=48, Hq=4, Hkv=2, d=16, theta=10000.0):
    q = _rand(rng, B, S, Hq, d)
    k = _rand(rng, B, S, Hkv, d)
    pos = np.arange(S)
    return O.apply_rope(q, pos, theta), O.apply_rope(k, pos, theta)


def pin_rows_sum_to_one():
    rng = np.random.default_rng(12)
    qr, kr = _rotated(rng)
    S = qr.shape[1]
    for causal in (True, False):
        P, _, _ = O.attention_weights(qr[0, :, 0], kr[0, :, 0], np.arange(S), causal)
        _close(P.sum(axis=-1), np.ones(S), 1e-12, f"row sums (causal={causal})")
        assert np.all(P >= 0.0), "negative softmax weight"


def pin_masked_exact_zero():
    rng = np.random.default_rng(13)
    qr, kr = _rotated(rng)
    S = qr.shape[1]
    P, _, _ = O.attention_weights(qr[0, :, 1], kr[0, :, 0], np.arange(S), True)
    future = np.triu(np.ones((S, S), dtype=bool), k=1)
    assert np.all(P[future] == 0.0), "a future key got non-zero weight"
    assert np.all(P[~future] > 0.0), "a visible key got zero weight"
    # Evaluating a subset of rows gives the same weights as the full matrix.
    rows = np.array([0, 5, S - 1])
    Pr, _, _ = O.attention_weights(qr[0, rows, 1], kr[0, :, 0], rows, True)
    _close(Pr, P[rows], 1e-15, "row subset of weights")


# ---------------------------------------------------------------- closed forms
def pin_row0_closed_form():
    rng = np.random.default_rng(14)
    B, S, Hq, Hkv, d = 2, 9, 4, 2, 8
    q = _rand(rng, B, S, Hq, d)
    k = _rand(rng, B, S, Hkv, d)
    v = _rand(rng, B, S, Hkv, d)
    out, lse = O.attention(q, k, v, 10000.0, causal=True)
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        _close(out[:, 0, h], v[:, 0, g], 1e-14, "row 0 out = v_0")
        _close(lse[:, h, 0], np.sum(q[:, 0, h] * k[:, 0, g], axis=-1) / math.sqrt(d), 1e-13,
               "row 0 lse = q_0.k_0/sqrt(d)")


def pin_zero_query():
    rng = np.random.default_rng(15)
    B, S, Hq, Hkv, d = 1, 12, 2, 1, 8
    q = np.zeros((B, S, Hq, d))
    k = _rand(rng, B, S, Hkv, d)
    v = _rand(rng, B, S, Hkv, d)
    out, lse = O.attention(q, k, v, 10000.0, causal=True)
    cummean = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, S + 1)[:, None]
    for h in range(Hq):
        _close(out[0, :, h], cummean, 1e-13, "q=0 causal out = running mean of v")
        _close(lse[0, h], np.log(np.arange(1, S + 1)), 1e-13, "q=0 causal lse = ln(i+1)")
    out, lse = O.attention(q, k, v, 10000.0, causal=False)
    _close(out[0, :, 0], np.broadcast_to(v[0, :, 0].mean(axis=0), (S, d)), 1e-13, "q=0 full out = mean v")
    _close(lse[0, 0], np.full(S, math.log(S)), 1e-13, "q=0 full lse = ln S")


def pin_constant_v():
    rng = np.random.default_rng(16)
    B, S, Hq, Hkv, d = 2, 10, 4, 2, 8
    q = _rand(rng, B, S, Hq, d)
    k = _rand(rng, B, S, Hkv, d)
    c = _rand(rng, B, 1, Hkv, d)
    v = np.broadcast_to(c, (B, S, Hkv, d)).copy()
    out, _ = O.attention(q, k, v, 10000.0, causal=True)
    G = Hq // Hkv
    for h in range(Hq):
        _close(out[:, :, h], np.broadcast_to(c[:, :, h // G], (B, S, d)), 1e-13, "constant v")


def pin_diagonal_dominance():
    rng = np.random.default_rng(17)
    B, S, H, d = 1, 16, 1, 8
    u = _rand(rng, B, S, H, d)
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    q = 40.0 * u
    k = 40.0 * u
    v = _rand(rng, B, S, H, d)
    out, _ = O.attention(q, k, v, 10000.0, causal=True)
    _close(out, v, 1e-9, "dominant diagonal picks v_i")


# ---------------------------------------------------------------- GQA
def pin_gqa_repeat():
    rng = np.random.default_rng(18)
    B, S, d = 1, 14, 8
    for (Hq, Hkv) in ((6, 2), (4, 1), (4, 4), (8, 2)):
        q = _rand(rng, B, S, Hq, d)
        k = _rand(rng, B, S, Hkv, d)
        v = _rand(rng, B, S, Hkv, d)
        G = Hq // Hkv
        out, lse = O.attention(q, k, v, 10000.0, causal=True)
        out_m, lse_m = O.attention(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), 10000.0, causal=True)
        _close(out, out_m, 1e-14, f"GQA {Hq}/{Hkv} vs repeated-head MHA out")
        _close(lse, lse_m, 1e-14, f"GQA {Hq}/{Hkv} vs repeated-head MHA lse")


# ---------------------------------------------------------------- rotation facts
def pin_rope_norm():
    rng = np.random.default_rng(19)
    x = _rand(rng, 2, 33, 3, 16)
    for theta in (10000.0, 500000.0):
        xr = O.apply_rope(x, np.arange(33), theta)
        _close(np.linalg.norm(xr, axis=-1), np.linalg.norm(x, axis=-1), 1e-12, "rotation keeps norm")
        xr = O.apply_rope(x[:, :1], np.array([32767]), theta)
        _close(np.linalg.norm(xr, axis=-1), np.linalg.norm(x[:, :1], axis=-1), 1e-12, "norm at p=32767")


def pin_rope_relative():
    rng = np.random.default_rng(20)
    d = 16
    q = _rand(rng, 1, 1, 1, d)
    k = _rand(rng, 1, 1, 1, d)
    for theta in (10000.0, 500000.0):
        for (p, pk) in ((3, 1), (0, 7), (100, 100), (2047, 5)):
            ref = np.sum(O.apply_rope(q, [p], theta) * O.apply_rope(k, [pk], theta))
            for t in (1, 17, 1000, 30000):
                got = np.sum(O.apply_rope(q, [p + t], theta) * O.apply_rope(k, [pk + t], theta))
                assert abs(got - ref) <= 1e-10 * (1 + abs(ref)), "q.k depends on more than p - p'"
            # and it does depend on the difference
            other = np.sum(O.apply_rope(q, [p + 1], theta) * O.apply_rope(k, [pk], theta))
            assert abs(other - ref) > 1e-9, "rotation had no effect on q.k"


def pin_rope_identity():
    rng = np.random.default_rng(21)
    x = _rand(rng, 2, 1, 3, 8)
    assert np.array_equal(O.apply_rope(x, [0], 10000.0), x), "rotation at position 0 is not the identity"


def pin_rope_d2_textbook():
    # For head_dim 2 the single frequency is theta**0 = 1, so position p rotates by p radians.
    rng = np.random.default_rng(22)
    x = _rand(rng, 1, 1, 1, 2)
    for p in (1, 2, 5, 1000):
        R = np.array([[math.cos(p), -math.sin(p)], [math.sin(p), math.cos(p)]])
        got = O.apply_rope(x, [p], 12345.0)[0, 0, 0]
        _close(got, R @ x[0, 0, 0], 1e-12, f"d=2 textbook rotation at p={p}")


def pin_rope_frequencies_llama3():
    # llama3 page, "RoPE principle": 1/rope_theta**(arange(64)/64) for head_dim 128.
    for theta in (10000.0, 500000.0):
        ref = np.array([1.0 / theta ** (i / 64.0) for i in range(64)])
        _close(O.rope_frequencies(128, theta), ref, 1e-15, "frequencies vs the llama3 page")


# ---------------------------------------------------------------- library routines
def pin_sdpa():
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(23)
    B, S, Hq, Hkv, d = 2, 37, 6, 2, 16
    q = _rand(rng, B, S, Hq, d)
    k = _rand(rng, B, S, Hkv, d)
    v = _rand(rng, B, S, Hkv, d)
    G = Hq // Hkv
    pos = np.arange(S)
    qr = torch.from_numpy(O.apply_rope(q, pos, 500000.0)).permute(0, 2, 1, 3)
    kr = torch.from_numpy(O.apply_rope(k, pos, 500000.0)).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    for causal in (True, False):
        ref = F.scaled_dot_product_attention(qr, kr, vt, is_causal=causal).permute(0, 2, 1, 3).numpy()
        out, _ = O.attention(q, k, v, 500000.0, causal=causal)
        _close(out, ref, 1e-12, f"SDPA float64 (causal={causal})")


def pin_lse_scipy():
    from scipy.special import logsumexp

    rng = np.random.default_rng(24)
    B, S, Hq, Hkv, d = 1, 29, 4, 1, 8
    q = _rand(rng, B, S, Hq, d, scale=2.0)
    k = _rand(rng, B, S, Hkv, d, scale=2.0)
    v = _rand(rng, B, S, Hkv, d)
    pos = np.arange(S)
    qr = O.apply_rope(q, pos, 10000.0)
    kr = O.apply_rope(k, pos, 10000.0)
    for causal in (True, False):
        _, lse = O.attention(q, k, v, 10000.0, causal=causal)
        for h in range(Hq):
            sc = np.einsum("ic,jc->ij", qr[0, :, h], kr[0, :, 0]) / math.sqrt(d)
            if causal:
                sc = np.where(np.tril(np.ones((S, S), dtype=bool)), sc, -np.inf)
            _close(lse[0, h], logsumexp(sc, axis=-1), 1e-12, f"lse vs scipy (causal={causal})")


# ---------------------------------------------------------------- other page's form
def _llama3_complex_rotate(x, positions, rope_theta):
    # llama3 page, "parallel rotation of queries and keys": adjacent pairs viewed as complex
    # numbers times polar(1, p * freq), freq = 1/rope_theta**(arange(d/2)/(d/2)).
    d = x.shape[-1]
    freqs = 1.0 / rope_theta ** (np.arange(d // 2) / (d // 2))
    ang = np.outer(positions, freqs)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * np.exp(1j * ang)[None, :, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def pin_interleaved_equivalence():
    rng = np.random.default_rng(25)
    B, S, Hq, Hkv, d = 1, 20, 4, 2, 16
    q = _rand(rng, B, S, Hq, d)
    k = _rand(rng, B, S, Hkv, d)
    v = _rand(rng, B, S, Hkv, d)
    theta = 500000.0
    pos = np.arange(S)
    qi = _llama3_complex_rotate(q, pos, theta)
    ki = _llama3_complex_rotate(k, pos, theta)
    G = Hq // Hkv
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    out_h, lse_h = O.attention(q[..., perm], k[..., perm], v, theta, causal=True)
    for h in range(Hq):
        g = h // G
        sc = qi[0, :, h] @ ki[0, :, g].T / math.sqrt(d)
        sc = np.where(np.tril(np.ones((S, S), dtype=bool)), sc, -np.inf)
        m = sc.max(axis=-1, keepdims=True)
        e = np.exp(sc - m)
        _close(out_h[0, :, h], (e / e.sum(-1, keepdims=True)) @ v[0, :, g], 1e-12,
               "interleaved complex form vs permuted half-split (out)")
        _close(lse_h[0, h], (m[:, 0] + np.log(e.sum(-1))), 1e-12,
               "interleaved complex form vs permuted half-split (lse)")
    # the oracle's own interleaved path: its rotation is the complex form, and its attention
    # equals the permuted half-split one
    _close(O.apply_rope_interleaved(q, pos, theta), qi, 1e-12, "apply_rope_interleaved vs complex form")
    out_i, lse_i = O.attention(q, k, v, theta, causal=True, interleaved=True)
    _close(out_i, out_h, 1e-12, "interleaved attention vs permuted half-split (out)")
    _close(lse_i, lse_h, 1e-12, "interleaved attention vs permuted half-split (lse)")


# ---------------------------------------------------------------- lse meaning
def pin_lse_merge():
    rng = np.random.default_rng(26)
    S, d = 40, 8
    qr, kr = _rotated(rng, S=S, d=d)
    v = _rand(rng, S, d)
    rows = np.arange(S)
    P, m, l = O.attention_weights(qr[0, :, 0], kr[0, :, 0], rows, False)
    full_out = P @ v
    full_lse = m + np.log(l)
    split = rng.permutation(S)
    a, b = split[:17], split[17:]
    Pa, ma, la = O.attention_weights(qr[0, :, 0], kr[0, a, 0], rows, False)
    Pb, mb, lb = O.attention_weights(qr[0, :, 0], kr[0, b, 0], rows, False)
    lse_a, lse_b = ma + np.log(la), mb + np.log(lb)
    lse = np.logaddexp(lse_a, lse_b)
    out = np.exp(lse_a - lse)[:, None] * (Pa @ v[a]) + np.exp(lse_b - lse)[:, None] * (Pb @ v[b])
    _close(lse, full_lse, 1e-12, "merged lse")
    _close(out, full_out, 1e-12, "merged out")


# ---------------------------------------------------------------- sequence shards
def pin_shard_shift_invariance():
    """Shifting query and key positions together changes nothing: RoPE scores depend only on
    the position difference and so does the causal mask."""
    rng = np.random.default_rng(31)
    q, k, v = _rand(rng, 1, 20, 4, 8), _rand(rng, 1, 20, 2, 8), _rand(rng, 1, 20, 2, 8)
    for causal in (True, False):
        o0, l0 = O.attention(q, k, v, 500.0, causal)
        o1, l1 = O.attention(q, k, v, 500.0, causal, q_pos0=37, k_pos0=37)
        _close(o1, o0, 1e-12, "shifted shard out")
        _close(l1, l0, 1e-12, "shifted shard lse")


def pin_ring_split():
    """Causal attention over S = 3 shards of queries, each merged over all 3 shards of keys at
    their offsets (later shards see nothing and must not change the merge)."""
    rng = np.random.default_rng(32)
    S, n = 48, 16
    q, k, v = _rand(rng, 2, S, 4, 8), _rand(rng, 2, S, 2, 8), _rand(rng, 2, S, 2, 8)
    full_o, full_l = O.attention(q, k, v, 10000.0, True)
    for s in range(3):
        qs = q[:, s * n:(s + 1) * n]
        o, l = None, None
        for t in range(3):
            ot, lt = O.attention(qs, k[:, t * n:(t + 1) * n], v[:, t * n:(t + 1) * n], 10000.0, True,
                                 q_pos0=s * n, k_pos0=t * n)
            if t > s:
                assert np.all(lt == -np.inf) and np.all(ot == 0.0), "a later key shard must be empty"
            o, l = (ot, lt) if o is None else O.merge(o, l, ot, lt)
        _close(o, full_o[:, s * n:(s + 1) * n], 1e-12, f"ring shard {s} out")
        _close(l, full_l[:, :, s * n:(s + 1) * n], 1e-12, f"ring shard {s} lse")


def pin_empty_rows():
    """Queries that precede every key: out exactly 0, lse exactly -inf; a partly visible shard
    equals the plain definition on its visible keys."""
    rng = np.random.default_rng(33)
    q, k, v = _rand(rng, 1, 12, 2, 4), _rand(rng, 1, 12, 1, 4), _rand(rng, 1, 12, 1, 4)
    o, l = O.attention(q, k, v, 100.0, True, q_pos0=0, k_pos0=12)
    assert np.all(o == 0.0) and np.all(l == -np.inf), "queries before every key"
    o, l = O.attention(q, k, v, 100.0, True, q_pos0=0, k_pos0=5)
    assert np.all(o[:, :5] == 0.0) and np.all(l[:, :, :5] == -np.inf), "rows 0-4 see no key"
    # row i >= 5 sees keys 0 .. i-5 of this shard: brute force with the page's formulas
    qr = O.apply_rope(q, np.arange(12), 100.0)
    kr = O.apply_rope(k, 5 + np.arange(12), 100.0)
    for i in range(5, 12):
        sc = kr[0, : i - 4, 0] @ qr[0, i, 0] / 2.0
        e = np.exp(sc - sc.max())
        _close(o[0, i, 0], (e / e.sum()) @ v[0, : i - 4, 0], 1e-12, f"partly visible row {i}")
        _close(l[0, 0, i], sc.max() + np.log(e.sum()), 1e-12, f"partly visible row {i} lse")


# ---------------------------------------------------------------- golden fixtures
def pin_golden():
    path = os.path.join(GOLDEN_DIR, "closed_form_cases.json")
    with open(path, "r", encoding="utf-8") as f:
        cases = json.load(f)["cases"]
    assert cases, "no golden cases"
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)
        k = np.array(c["k"], dtype=np.float64)
        v = np.array(c["v"], dtype=np.float64)
        out, lse = O.attention(q, k, v, c["rope_theta"], causal=c["causal"])
        _close(out, np.array(c["out"]), 1e-14, f"golden {c['name']} out")
        _close(lse, np.array(c["lse"]), 1e-14, f"golden {c['name']} lse")


BACKWARD_FD_CASES = [
    # B, S, Hq, Hkv, d, causal, rope_theta, seed, interleaved
    (1, 5, 2, 1, 4, True, 100.0, 1, False),
    (2, 4, 2, 2, 6, False, 10.0, 2, False),
    (1, 6, 3, 1, 8, True, 10000.0, 3, False),
    (1, 3, 4, 2, 2, True, 3.0, 4, False),
    (1, 5, 2, 1, 6, True, 20.0, 5, True),
]


def pin_backward_finite_differences():
    """dq, dk, dv against central differences of L = sum(dout * out) through the forward."""
    h = 1e-6
    for B, S, Hq, Hkv, d, causal, theta, seed, il in BACKWARD_FD_CASES:
        rng = np.random.default_rng(seed)
        q, k, v = _rand(rng, B, S, Hq, d), _rand(rng, B, S, Hkv, d), _rand(rng, B, S, Hkv, d)
        do = _rand(rng, B, S, Hq, d)
        grads = dict(zip("qkv", O.attention_backward(q, k, v, do, theta, causal, interleaved=il)))
        x = {"q": q, "k": k, "v": v}
        for name in "qkv":
            num = np.zeros_like(x[name])
            for idx in np.ndindex(x[name].shape):
                args = dict(x)
                xp = x[name].copy()
                xp[idx] += h
                args[name] = xp
                lp = (O.attention(args["q"], args["k"], args["v"], theta, causal, interleaved=il)[0] * do).sum()
                xm = x[name].copy()
                xm[idx] -= h
                args[name] = xm
                lm = (O.attention(args["q"], args["k"], args["v"], theta, causal, interleaved=il)[0] * do).sum()
                num[idx] = (lp - lm) / (2 * h)
            _close(grads[name], num, 1e-7, f"d{name} vs finite differences, case seed {seed}")


def pin_backward_dv_sums_to_dout():
    """sum over keys of dv[:, :, g] = sum over the group's query heads and rows of dout."""
    rng = np.random.default_rng(31)
    B, S, Hq, Hkv, d = 2, 40, 6, 2, 16
    q, k, v = _rand(rng, B, S, Hq, d), _rand(rng, B, S, Hkv, d), _rand(rng, B, S, Hkv, d)
    do = _rand(rng, B, S, Hq, d)
    for causal in (True, False):
        _, _, dv = O.attention_backward(q, k, v, do, 500.0, causal)
        want = do.reshape(B, S, Hkv, Hq // Hkv, d).sum(axis=(1, 3))
        _close(dv.sum(axis=1), want, 1e-10, f"dv column sums, causal {causal}")


def pin_backward_row0_dq_zero():
    """Causal row 0 attends to key 0 alone: its softmax weight is 1 whatever the score, so
    dq[:, 0] is exactly 0 (up to rounding), while later rows are not."""
    rng = np.random.default_rng(32)
    q, k, v = _rand(rng, 1, 12, 4, 8), _rand(rng, 1, 12, 2, 8), _rand(rng, 1, 12, 2, 8)
    do = _rand(rng, 1, 12, 4, 8)
    dq, _, _ = O.attention_backward(q, k, v, do, 10000.0, True)
    assert np.abs(dq[:, 0]).max() < 1e-12, "causal dq row 0 must vanish"
    assert np.abs(dq[:, 1:]).max() > 1e-3, "later dq rows must not vanish"


def pin_backward_shard_single_block():
    """One block holding the whole sequence, with the forward's own out and lse, is the plain
    backward."""
    rng = np.random.default_rng(41)
    q, k, v = _rand(rng, 2, 24, 4, 8), _rand(rng, 2, 24, 2, 8), _rand(rng, 2, 24, 2, 8)
    do = _rand(rng, 2, 24, 4, 8)
    for causal, il in ((True, False), (False, False), (True, True)):
        out, lse = O.attention(q, k, v, 300.0, causal, interleaved=il)
        got = O.attention_backward_shard(q, k, v, do, out, lse, 300.0, causal, interleaved=il)
        want = O.attention_backward(q, k, v, do, 300.0, causal, interleaved=il)
        for n, a, b in zip("qkv", got, want):
            _close(a, b, 1e-12, f"single-block shard d{n}, causal {causal}, interleaved {il}")


def pin_backward_ring_split():
    """The backward of ring attention: split the sequence into 3 blocks; each (query block, key
    block) step at its offsets, with the full forward's out and lse for its queries, gives a part
    of the gradients; dq summed over key blocks and dk, dv summed over query blocks equal the
    plain backward of the whole sequence (finite-difference pinned)."""
    rng = np.random.default_rng(42)
    S, n = 48, 16
    for causal, il in ((True, False), (False, False), (True, True)):
        q, k, v = _rand(rng, 1, S, 4, 8), _rand(rng, 1, S, 2, 8), _rand(rng, 1, S, 2, 8)
        do = _rand(rng, 1, S, 4, 8)
        out, lse = O.attention(q, k, v, 1000.0, causal, interleaved=il)
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for a in range(3):
            qa = slice(a * n, (a + 1) * n)
            for c in range(3):
                kc = slice(c * n, (c + 1) * n)
                gq, gk, gv = O.attention_backward_shard(q[:, qa], k[:, kc], v[:, kc], do[:, qa], out[:, qa],
                                                        lse[:, :, qa], 1000.0, causal, q_pos0=a * n, k_pos0=c * n,
                                                        interleaved=il)
                if causal and c > a:
                    assert not gq.any() and not gk.any() and not gv.any(), "a later key block has no gradient"
                dq[:, qa] += gq
                dk[:, kc] += gk
                dv[:, kc] += gv
        want = O.attention_backward(q, k, v, do, 1000.0, causal, interleaved=il)
        for nm, a_, b_ in zip("qkv", (dq, dk, dv), want):
            _close(a_, b_, 1e-12, f"ring backward d{nm}, causal {causal}, interleaved {il}")


def pin_backward_shard_shift_invariance():
    """Moving both blocks by the same number of positions changes no gradient: the scores and
    the mask depend on position differences, and each rotation back undoes its own angle."""
    rng = np.random.default_rng(43)
    q, k, v = _rand(rng, 1, 20, 2, 8), _rand(rng, 1, 20, 1, 8), _rand(rng, 1, 20, 1, 8)
    do = _rand(rng, 1, 20, 2, 8)
    out, lse = O.attention(q, k, v, 700.0, True, q_pos0=21, k_pos0=30)
    g0 = O.attention_backward_shard(q, k, v, do, out, lse, 700.0, True, q_pos0=21, k_pos0=30)
    out1, lse1 = O.attention(q, k, v, 700.0, True, q_pos0=21 + 55, k_pos0=30 + 55)
    g1 = O.attention_backward_shard(q, k, v, do, out1, lse1, 700.0, True, q_pos0=21 + 55, k_pos0=30 + 55)
    for n, a, b in zip("qkv", g0, g1):
        _close(a, b, 1e-12, f"shifted shard d{n}")
    # rows 0..8 see no key of this block (their lse is -inf): no gradient flows through them,
    # and keys 11.. are seen by no row
    assert np.all(lse[:, :, :9] == -np.inf) and np.isfinite(lse[:, :, 9:]).all()
    assert not g0[0][:, :9].any() and np.abs(g0[0][:, 9:]).max() > 1e-3
    assert not g0[1][:, 11:].any() and not g0[2][:, 11:].any()


ALL_PINS = [
    pin_bruteforce,
    pin_rows_sum_to_one,
    pin_masked_exact_zero,
    pin_row0_closed_form,
    pin_zero_query,
    pin_constant_v,
    pin_diagonal_dominance,
    pin_gqa_repeat,
    pin_rope_norm,
    pin_rope_relative,
    pin_rope_identity,
    pin_rope_d2_textbook,
    pin_rope_frequencies_llama3,
    pin_sdpa,
    pin_lse_scipy,
    pin_interleaved_equivalence,
    pin_lse_merge,
    pin_shard_shift_invariance,
    pin_ring_split,
    pin_empty_rows,
    pin_backward_finite_differences,
    pin_backward_dv_sums_to_dout,
    pin_backward_row0_dq_zero,
    pin_backward_shard_single_block,
    pin_backward_ring_split,
    pin_backward_shard_shift_invariance,
    pin_golden,
]
