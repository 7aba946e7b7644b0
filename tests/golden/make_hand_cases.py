"""Write ``hand_cases.json``: tiny attention problems whose outputs were derived by hand.

The pages print no numeric worked example, so these cases are small enough to
solve on paper from the definition S = scale * Q K^T (+ bias), P = softmax(S),
O = P V, lse = log sum exp(S) ("FlashAttention: Faster Attention Without
Dropping a Single Interaction", Method Deep Dive, Key design 1 and its
saved-state table) and the backward of Key design 3. This script only evaluates
the closed forms written below with ``math``; it calls no implementation of
attention.

Run from the repository root: ``python tests/golden/make_hand_cases.py``.
"""

import json
import math
import os

E = math.e


def case_two_keys():
    # d = 1, scale = 1, q = k = [[1], [0]], v = [[2], [4]], dO = [[1], [0]].
    # S = [[1, 0], [0, 0]]; P_0 = [e, 1] / (1 + e); P_1 = [1/2, 1/2].
    o0 = (2 * E + 4) / (1 + E)
    p00 = E / (1 + E)
    # loss = O_0: dV_j = P_0j; dP_0j = v_j, D_0 = O_0, dS_0j = P_0j (v_j - O_0).
    # dQ_0 = dS_00 * k_0 + dS_01 * k_1 = P_00 (2 - O_0) = -2e / (1 + e)^2.
    ds00 = p00 * (2 - o0)
    ds01 = (1 - p00) * (4 - o0)
    return {
        "name": "two_keys",
        "derivation": "S=[[1,0],[0,0]]; O_0=(2e+4)/(1+e), O_1=3; lse=[ln(1+e), ln 2]; "
                      "dV=[e/(1+e), 1/(1+e)]; dQ_0=-2e/(1+e)^2, dQ_1=0; dK_j = dS_0j q_0",
        "scale": 1.0, "causal": False, "alibi_slopes": None,
        "q": [[[[1.0]], [[0.0]]]], "k": [[[[1.0]], [[0.0]]]], "v": [[[[2.0]], [[4.0]]]],
        "do": [[[[1.0]], [[0.0]]]],
        "o": [[[[o0]], [[3.0]]]],
        "lse": [[[math.log(1 + E), math.log(2.0)]]],
        "dq": [[[[-2 * E / (1 + E) ** 2]], [[0.0]]]],
        "dk": [[[[ds00 * 1.0]], [[ds01 * 1.0]]]],
        "dv": [[[[p00]], [[1 - p00]]]],
    }


def case_alibi_causal():
    # d = 1, q = k = 0 so S is the bias alone: S_ij = -(i - j) for j <= i, slope 1.
    # v = [[1], [2], [3]]. Row i: weights e^{-(i-j)}, j = 0..i.
    o, lse = [], []
    for i in range(3):
        w = [math.exp(-(i - j)) for j in range(i + 1)]
        z = sum(w)
        o.append([[sum(wj * (j + 1) for j, wj in enumerate(w)) / z]])
        lse.append(math.log(z))
    return {
        "name": "alibi_causal",
        "derivation": "q=k=0, slope 1, causal: S_ij=-(i-j); O_2=(e^-2+2e^-1+3)/(1+e^-1+e^-2), "
                      "lse_2=ln(1+e^-1+e^-2); row 0 copies v_0",
        "scale": 1.0, "causal": True, "alibi_slopes": [1.0],
        "q": [[[[0.0]], [[0.0]], [[0.0]]]], "k": [[[[0.0]], [[0.0]], [[0.0]]]],
        "v": [[[[1.0]], [[2.0]], [[3.0]]]],
        "o": [o],
        "lse": [[lse]],
    }


if __name__ == "__main__":
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "hand_cases.json"), "w") as f:
        json.dump({"cases": [case_two_keys(), case_alibi_causal()]}, f)
        f.write("\n")
