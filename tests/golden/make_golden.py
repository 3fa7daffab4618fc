"""Writes ``exact_small.json``: tiny KDA cases solved in exact rational arithmetic.

Calls only ``oracle.exact``. Inputs are dyadic rationals (exact in fp32); alpha is taken as the
exact binary value of exp(log_alpha) for an fp32 log_alpha, so the stored outputs are the exact
result of the recurrence in section 2.2 of the Kimi K3 reading notes
(liuzhao09.github.io/papers/kimi-k3.html) for those inputs. Run: python tests/golden/make_golden.py
"""
import json
import math
import os
import random
import sys
from fractions import Fraction

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import exact  # noqa: E402


def _case(seed, T, dk, dv, with_s0):
    rnd = random.Random(seed)
    dy = lambda den, lo, hi: Fraction(rnd.randint(int(lo * den), int(hi * den)), den)
    q = [[dy(8, -1, 1) for _ in range(dk)] for _ in range(T)]
    k = [[dy(8, -1, 1) for _ in range(dk)] for _ in range(T)]
    v = [[dy(8, -2, 2) for _ in range(dv)] for _ in range(T)]
    beta = [Fraction(rnd.randint(1, 15), 16) for _ in range(T)]
    la = [[float(np.float32(-rnd.randint(0, 64) / 128.0 - rnd.random() * 0.01)) for _ in range(dk)] for _ in range(T)]
    alpha = [[Fraction(math.exp(x)) for x in row] for row in la]
    S0 = [[dy(16, -1, 1) for _ in range(dv)] for _ in range(dk)] if with_s0 else None
    o, S = exact.kda_fwd(q, k, v, alpha, beta, S0)
    f = lambda m: [[float(x) for x in row] for row in m]
    s = lambda m: [[str(x) for x in row] for row in m]
    return {"seed": seed, "T": T, "dk": dk, "dv": dv,
            "q": f(q), "k": f(k), "v": f(v), "beta": [float(b) for b in beta], "log_alpha": la,
            "S0": f(S0) if S0 else None, "o": s(o), "S_T": s(S)}


def main():
    cases = [_case(1, 6, 2, 2, False), _case(2, 9, 3, 2, True), _case(3, 12, 4, 3, True), _case(4, 16, 3, 4, False)]
    doc = {"citation": "Kimi K3 reading notes (liuzhao09.github.io/papers/kimi-k3.html), section 2.2, "
                       "KDA state recurrence S_t=(I-beta_t k_t k_t^T)Diag(alpha_t)S_{t-1}+beta_t k_t v_t^T, "
                       "o_t=S_t^T q_t; alpha=exp(log_alpha) evaluated once in fp64 and then treated as exact",
           "generator": "tests/golden/make_golden.py (oracle.exact only)", "cases": cases}
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exact_small.json")
    with open(out, "w") as fh:
        json.dump(doc, fh, indent=1)
    print("wrote", out)


if __name__ == "__main__":
    main()
