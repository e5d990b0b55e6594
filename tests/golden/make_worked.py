"""Writes the hand-derived worked examples in this folder.

Every expected value here is a closed form derived by hand from the
definitions in the TokenGate paper, Section 4 (each JSON file carries its
derivation and citation); the script evaluates those closed forms with the
``math`` module only.  It calls neither the oracle nor the HIP library.
Run: python tests/golden/make_worked.py
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def silu(x):
    return x / (1.0 + math.exp(-x))


def main():
    e = math.e
    s2, s1 = silu(2.0), silu(1.0)
    score = {
        "source": "TokenGate paper, Section 4, 'Scoring Network' (Eq. 1 row RMSNorm, Eq. 3 scoring MLP); "
                  "workload shapes name the activation 'd->h->1 SiLU'.",
        "derivation": [
            "eps_row = 0, norm weight w = [2, 0.5], W1 = [[1,0],[0,2],[-1,-2]], b1 = [0,0,1], w2 = [1,-1,2], b2 = 0.25, r = 1.",
            "Row 0 is non-prunable (j < r): score fixed to 0 whatever its values.",
            "Row 1, a = [1, 1]: mean square 1, normalised [2, 0.5], u = [2, 1, -2]; silu(-2) = silu(2) - 2, "
            "so b~ = silu(2) - silu(1) + 2 silu(-2) + 0.25 = 3 silu(2) - silu(1) - 3.75.",
            "Row 2, a = [2, 2]: same direction, RMSNorm removes the scale, so b~ equals row 1's.",
            "Row 3, a = [3, -3]: normalised [2, -0.5], u = [2, -1, 0]; silu(-1) = silu(1) - 1, silu(0) = 0, "
            "so b~ = silu(2) - silu(1) + 1 + 0.25.",
            "silu(x) = x / (1 + exp(-x)).",
        ],
        "r": 1, "eps_row": 0.0,
        "resid": [[[5.0, -7.0], [1.0, 1.0], [2.0, 2.0], [3.0, -3.0]]],
        "norm_w": [2.0, 0.5], "W1": [[1.0, 0.0], [0.0, 2.0], [-1.0, -2.0]], "b1": [0.0, 0.0, 1.0],
        "w2": [1.0, -1.0, 2.0], "b2": [0.25],
        "expected": [[0.0, 3 * s2 - s1 - 3.75, 3 * s2 - s1 - 3.75, s2 - s1 + 1.25]],
    }
    seq = {
        "source": "TokenGate paper, Section 4, 'Scoring Network' (Eq. 3: scores RMS-normalised along the "
                  "sequence, fixed to 0 on non-prunable tokens).",
        "derivation": [
            "r = 1, eps_seq = 0; the raw score of the non-prunable token (7) is ignored and its output is 0.",
            "Prunable raw scores [3, -4]: mean square over the prunable span (9 + 16) / 2 = 12.5, so "
            "b = [3, -4] / sqrt(12.5) = [0.6 sqrt(2), -0.8 sqrt(2)].",
        ],
        "r": 1, "eps_seq": 0.0, "score_raw": [[7.0, 3.0, -4.0]],
        "expected": [[0.0, 0.6 * math.sqrt(2), -0.8 * math.sqrt(2)]],
    }
    topk = {
        "source": "TokenGate paper, Section 4, 'Top-K Selector' (Eq. 4: the K highest-scoring prunable tokens "
                  "plus every non-prunable token). Tie and NaN rules are this implementation's reading.",
        "derivation": [
            "Scores [5, 1, 3, 3, NaN, -inf, 2] with r = 1: token 0 is always kept.",
            "Prunable order (score desc, index asc, NaN last): 2 (3), 3 (3), 6 (2), 1 (1), 5 (-inf), 4 (NaN).",
            "K = 3 keeps 2, 3, 6; K = 5 adds 1 and 5; K = 6 or more keeps all; K = 0 keeps only token 0.",
        ],
        "r": 1, "score": [[5.0, 1.0, 3.0, 3.0, "nan", "-inf", 2.0]],
        "cases": {"0": [[1, 0, 0, 0, 0, 0, 0]], "3": [[1, 0, 1, 1, 0, 0, 1]], "5": [[1, 1, 1, 1, 0, 1, 1]],
                  "6": [[1, 1, 1, 1, 1, 1, 1]], "9": [[1, 1, 1, 1, 1, 1, 1]]},
    }
    se = math.sqrt(e)
    attn = {
        "source": "TokenGate paper, Section 4: token-gated attention (Eq. 5), 'Head-wise' gate (Eq. 6), "
                  "'Temperature Scaling' (Eq. 7, log-ratio reading), 'Putting everything together' (Eq. 8).",
        "derivation": [
            "One head, d_h = 1, sm_scale = 1, gain = 1, temp = 1; q = [1, 1], k = [1, 2], v = [10, 20], b = [0, ln 2].",
            "Row 0 sees only key 0: O_0 = 10, lse_0 = q0 k0 + b0 = 1.",
            "Row 1 with pos = [0, 1] (full context, ratio 1): logits [1, 2 + ln 2], weights proportional to "
            "[e, 2 e^2]: O_1 = (10 + 40 e) / (1 + 2 e), lse_1 = 1 + ln(1 + 2 e).",
            "Row 1 with pos = [0, 3]: p = 4 keys at full context, m = 2 kept, ratio ln 4 / ln 2 = 2, so the QK "
            "logit is halved and the bias is not: logits [0.5, 1 + ln 2], weights proportional to [e^0.5, 2 e]: "
            "O_1 = (10 + 40 e^0.5) / (1 + 2 e^0.5), lse_1 = 0.5 + ln(1 + 2 e^0.5).",
        ],
        "q": [1.0, 1.0], "k": [1.0, 2.0], "v": [10.0, 20.0], "b": [0.0, math.log(2.0)],
        "cases": [
            {"pos": [0, 1], "O": [10.0, (10 + 40 * e) / (1 + 2 * e)], "lse": [1.0, 1 + math.log(1 + 2 * e)]},
            {"pos": [0, 3], "O": [10.0, (10 + 40 * se) / (1 + 2 * se)], "lse": [1.0, 0.5 + math.log(1 + 2 * se)]},
        ],
    }
    rope = rope_worked()
    for name, obj in [("score_worked", score), ("seqnorm_worked", seq), ("topk_worked", topk),
                      ("attention_worked", attn), ("rope_attention_worked", rope)]:
        with open(os.path.join(HERE, name + ".json"), "w") as f:
            json.dump(obj, f, indent=1)


def rope_worked():
    """Rotary attention at the original positions, d_h = 2 (one pair, angle pos
    radians at any base), through the relative-angle identity."""
    q = [[1.0, 0.0], [2.0, 1.0], [0.0, 2.0]]
    k = [[1.0, 1.0], [1.0, -1.0], [2.0, 0.0]]
    v = [[1.0, 0.0], [0.0, 1.0], [3.0, -2.0]]
    b = [0.0, 1.0, -1.0]
    pos = [0, 2, 5]
    gain = 0.5

    def s_rel(a, c, delta):
        # q_i R(pos_i) . k_j R(pos_j) = (a.c) cos(delta) + (a2 c1 - a1 c2) sin(delta), delta = pos_j - pos_i
        return (a[0] * c[0] + a[1] * c[1]) * math.cos(delta) + (a[1] * c[0] - a[0] * c[1]) * math.sin(delta)

    O, lse = [], []
    for i in range(3):
        ratio = 1.0 if pos[i] == i else math.log(max(pos[i] + 1, 2)) / math.log(max(i + 1, 2))
        z = [s_rel(q[i], k[j], pos[j] - pos[i]) / ratio + gain * b[j] for j in range(i + 1)]
        mx = max(z)
        w = [math.exp(x - mx) for x in z]
        tot = sum(w)
        O.append([sum(w[j] * v[j][c] for j in range(i + 1)) / tot for c in range(2)])
        lse.append(mx + math.log(tot))
    return {
        "source": "TokenGate paper, Appendix C.4 (kept tokens keep their original positions for the position "
                  "encoding) with Section 4, Eq. 8 and the Eq. 7 log-ratio reading; rotate-half rotary embedding "
                  "(pair (x_i, x_{i + d/2}) turned by pos * base^(-2i/d)).",
        "derivation": [
            "One head, d_h = 2: the single pair turns by pos radians (base^0 = 1), so the base does not matter.",
            "R(t) (x1, x2) = (x1 cos t - x2 sin t, x2 cos t + x1 sin t); R(a)^T R(b) = R(b - a), so "
            "R(p_i) q . R(p_j) k = (q.k) cos(p_j - p_i) + (q2 k1 - q1 k2) sin(p_j - p_i).",
            "z_ij = that product * sm_scale / (temp * ratio_i) + gain * b_j with sm_scale = temp = 1, gain = 0.5; "
            "ratio_0 = 1 (pos 0 = rank 0), ratio_1 = ln 3 / ln 2, ratio_2 = ln 6 / ln 3.",
            "O_i = sum_j softmax_j(z_i) v_j and lse_i = ln sum_j exp z_ij over j <= i.",
            "The oracle rounds the rotated q and k to bf16 (relative error <= 2^-9 per element): with |q|, |k| <= "
            "2.3 every logit moves by at most ~0.02, so O and lse agree to 0.05.",
        ],
        "q": q, "k": k, "v": v, "b": b, "pos": pos, "gain": gain, "base": 10000.0, "tol": 0.05,
        "O": O, "lse": lse,
    }


if __name__ == "__main__":
    main()
