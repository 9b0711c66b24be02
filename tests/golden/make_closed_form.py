"""Write closed_form_cases.json: tiny attention cases whose answers are derived by hand.

The pages print no numeric outputs, so these fixtures are closed forms instead: head_dim 2,
where the only rotation frequency is rope_theta**0 = 1 and position p turns a pair by p
radians, and two tokens, so every score can be written out.  Only the `math` module is used
here; nothing calls the oracle or the GPU path.

Definitions followed (the same the oracle cites):
  rotation: Picotron page, section 1 (x*cos + rotate_half(x)*sin), PaLM page section 2.3
            (frequencies 1/base**(arange(0, dim, 2)/dim));
  scores:   llama3 page, "attention score matrix" (q_rot . k_rot / sqrt(head_dim));
  mask:     llama3 page, "causal mask" (key j > query i gets -inf);
  softmax:  llama3 page "softmax" and PaLM page section 2.5;
  lse:      natural log of the softmax denominator (the form ring-style merging needs).

Run:  python tests/golden/make_closed_form.py
"""

import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))

C1, S1 = math.cos(1.0), math.sin(1.0)
R2 = math.sqrt(2.0)


def softmax2(s0, s1, v0, v1):
    w0, w1 = math.exp(s0), math.exp(s1)
    z = w0 + w1
    return [(w0 * a + w1 * b) / z for a, b in zip(v0, v1)], math.log(z)


def two_tokens(causal):
    # q0 = (1,0), q1 = (0,1); k0 = (1,0), k1 = (1,0); v0 = (1,2), v1 = (3,4); one head.
    # Position 0 is unrotated; position 1 turns by 1 rad:
    #   q1' = (-sin1, cos1), k1' = (cos1, sin1), k0' = k0, q0' = q0.
    # Row 0: s00 = 1/sqrt2, s01 = cos1/sqrt2.   Row 1: s10 = -sin1/sqrt2, s11 = 0.
    v0, v1 = [1.0, 2.0], [3.0, 4.0]
    if causal:
        out0, lse0 = v0, 1.0 / R2
    else:
        out0, lse0 = softmax2(1.0 / R2, C1 / R2, v0, v1)
    out1, lse1 = softmax2(-S1 / R2, 0.0, v0, v1)
    return {
        "name": "two_tokens_d2_" + ("causal" if causal else "full"),
        "derivation": "q0=(1,0) q1=(0,1) k0=k1=(1,0) v0=(1,2) v1=(3,4); d=2 so position p "
                      "rotates by p rad; row0 scores 1/sqrt2 (and cos1/sqrt2 if full); row1 "
                      "scores -sin1/sqrt2 and 0",
        "rope_theta": 10000.0,
        "causal": causal,
        "q": [[[[1.0, 0.0]], [[0.0, 1.0]]]],
        "k": [[[[1.0, 0.0]], [[1.0, 0.0]]]],
        "v": [[[v0], [v1]]],
        "out": [[[out0], [out1]]],
        "lse": [[[lse0, lse1]]],
    }


def mqa_two_heads():
    # Two query heads over one K/V head.  Head 0 is the causal two-token case above.
    # Head 1: q0 = (0,1), q1 = (1,0).  Row 0: s = q0.k0/sqrt2 = 0 (only key 0 visible).
    # Row 1: q1' = (cos1, sin1); s10 = cos1/sqrt2, s11 = (cos1^2 + sin1^2)/sqrt2 = 1/sqrt2.
    base = two_tokens(True)
    v0, v1 = [1.0, 2.0], [3.0, 4.0]
    out1_h1, lse1_h1 = softmax2(C1 / R2, 1.0 / R2, v0, v1)
    return {
        "name": "two_tokens_d2_mqa_causal",
        "derivation": "head0 as two_tokens_d2_causal; head1 q0=(0,1) q1=(1,0): row0 score 0, "
                      "row1 scores cos1/sqrt2 and 1/sqrt2; both heads read K/V head 0",
        "rope_theta": 500000.0,
        "causal": True,
        "q": [[[[1.0, 0.0], [0.0, 1.0]], [[0.0, 1.0], [1.0, 0.0]]]],
        "k": base["k"],
        "v": base["v"],
        "out": [[[base["out"][0][0][0], v0], [base["out"][0][1][0], out1_h1]]],
        "lse": [[base["lse"][0][0], [0.0, lse1_h1]]],
    }


def main():
    doc = {
        "source": "hand-derived closed forms (head_dim 2, two tokens); see make_closed_form.py",
        "cases": [two_tokens(True), two_tokens(False), mqa_two_heads()],
    }
    with open(os.path.join(HERE, "closed_form_cases.json"), "w", encoding="utf-8") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
