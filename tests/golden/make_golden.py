"""Writes tiny_recurrence.json: a small worked example of the GLA recurrence
(page "Gated Linear Attention (GLA) ...", section "The Gated Recurrent
Update"), evaluated by the fp64 oracle and nothing else.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

# T = 4 tokens, d_k = 2, d_v = 3; alpha is given as small fractions and g = log(alpha)
ALPHA = [[0.5, 1.0], [0.25, 0.5], [1.0, 0.125], [0.75, 0.5]]
Q = [[1.0, 2.0], [-1.0, 0.5], [2.0, -1.0], [0.0, 1.0]]
K = [[1.0, 0.0], [0.5, 1.0], [-1.0, 2.0], [1.0, 1.0]]
V = [[1.0, 2.0, 3.0], [0.0, -1.0, 1.0], [2.0, 0.0, -2.0], [1.0, 1.0, 1.0]]
S0 = [[0.5, 0.0, -0.5], [1.0, 1.0, 0.0]]


def main():
    g = np.log(np.array(ALPHA, dtype=np.float32)).astype(np.float32)
    q, k, v = (np.array(x, dtype=np.float32) for x in (Q, K, V))
    out = {"citation": "page 1, 'The Gated Recurrent Update': S_t = diag(alpha_t) S_{t-1} + k_t^T v_t, o_t = q_t S_t",
           "g_float32": g.tolist(), "q": Q, "k": K, "v": V, "s0": S0, "cases": {}}
    for name, s0 in (("zero_state", None), ("with_state", np.array(S0))):
        o, sf = oracle.recurrence(q[None, None], k[None, None], v[None, None], g[None, None],
                                  s0=None if s0 is None else s0[None, None])
        out["cases"][name] = {"o": o[0, 0].tolist(), "s_final": sf[0, 0].tolist()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_recurrence.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
