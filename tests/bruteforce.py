"""Pure-Python brute force for tiny attention problems (no numpy, no torch).

Deliberately takes a different route from the oracle wherever the mathematics allows, so a
slip in one is not repeated in the other:
  * the rotation of pair (c, c + d/2) is done as a complex product
    (x_c + i x_{c+d/2}) * exp(i * p * rope_theta**(-2c/d)), one element at a time;
  * the softmax has no max subtraction: weights are exp(score) / sum exp(score)
    (fine for the small magnitudes used here) and lse = log(sum exp(score));
  * the K/V head of query head h is found as floor(h * Hkv / Hq).
Inputs are nested Python lists q[b][s][h][c].
"""

import cmath
import math


def _rotate(x, pos, rope_theta):
    d = len(x)
    half = d // 2
    out = [0.0] * d
    for c in range(half):
        w = rope_theta ** (-2.0 * c / d)
        z = complex(x[c], x[c + half]) * cmath.exp(1j * pos * w)
        out[c] = z.real
        out[c + half] = z.imag
    return out


def brute_attention(q, k, v, rope_theta, causal):
    B = len(q)
    S = len(q[0])
    Hq = len(q[0][0])
    d = len(q[0][0][0])
    Hkv = len(k[0][0])
    out = [[[[0.0] * d for _ in range(Hq)] for _ in range(S)] for _ in range(B)]
    lse = [[[0.0] * S for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = (h * Hkv) // Hq
            krot = [_rotate(k[b][j][g], j, rope_theta) for j in range(S)]
            for i in range(S):
                qi = _rotate(q[b][i][h], i, rope_theta)
                keys = [j for j in range(S) if (not causal) or j <= i]
                w = []
                for j in keys:
                    dot = 0.0
                    for c in range(d):
                        dot += qi[c] * krot[j][c]
                    w.append(math.exp(dot / math.sqrt(d)))
                z = sum(w)
                for c in range(d):
                    acc = 0.0
                    for wj, j in zip(w, keys):
                        acc += wj * v[b][j][g][c]
                    out[b][i][h][c] = acc / z
                lse[b][h][i] = math.log(z)
    return out, lse
