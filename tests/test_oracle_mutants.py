"""Planted mistakes, on the CPU: each mutated copy of the oracle's arithmetic must fail at least
one of the pins used for the real oracle. This shows the pins can tell a plausible slip
(dropped term, wrong order, transposed operand, wrong triangle) from the recurrence of
section 2.2 of the Kimi K3 reading notes (liuzhao09.github.io/papers/kimi-k3.html)."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import native

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _loop(q, k, v, la, beta, S0, variant):
    q, k, v, la, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, la, beta))
    L, T, dk = q.shape
    dv = v.shape[2]
    S = np.zeros((L, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.zeros((L, T, dv))
    for t in range(T):
        a = np.exp(la[:, t])[:, :, None]
        kt, qt, vt, bt = k[:, t], q[:, t], v[:, t], beta[:, t, None, None]
        if variant == "read_before_write":
            o[:, t] = np.einsum("lc,lcj->lj", qt, a * S)
        if variant == "predict_undecayed":           # the simplified page-4 form
            pred = np.einsum("lc,lcj->lj", kt, S)
            S = a * S
        elif variant == "decay_after_write":
            pred = np.einsum("lc,lcj->lj", kt, S)
        else:
            S = a * S
            pred = np.einsum("lc,lcj->lj", kt, S)
        if variant == "no_beta_in_erase":
            S = S - kt[:, :, None] * pred[:, None, :] + bt * kt[:, :, None] * vt[:, None, :]
        else:
            S = S + bt * kt[:, :, None] * (vt[:, None, :] - pred[:, None, :])
        if variant == "decay_after_write":
            S = a * S
        if variant == "transposed_read":
            o[:, t] = np.einsum("lj,lcj->lc", qt, S)
        elif variant != "read_before_write":
            o[:, t] = np.einsum("lc,lcj->lj", qt, S)
    return o, S


def _chunk_mutant(q, k, v, la, beta, S0, variant, C=16):
    from scipy.linalg import solve_triangular
    q, k, v, la, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, la, beta))
    L, T, dk = q.shape
    o = np.zeros((L, T, v.shape[2]))
    Sout = []
    for l in range(L):
        S = np.array(S0[l], dtype=np.float64)
        for s in range(0, T, C):
            e = min(T, s + C)
            G = np.cumsum(la[l, s:e], axis=0)
            Gam = np.exp(G)
            Kg, Kinv = k[l, s:e] * Gam, k[l, s:e] / Gam
            Kbar = k[l, s:e] * (Gam if variant == "kbar_forward_decay" else np.exp(G[-1] - G))
            A_kk = beta[l, s:e, None] * np.tril(Kg @ Kinv.T, -1 if variant != "akk_with_diag" else 0)
            IA = np.eye(e - s) + A_kk
            U = solve_triangular(IA, beta[l, s:e, None] * v[l, s:e], lower=True)
            W = solve_triangular(IA, beta[l, s:e, None] * Kg, lower=True)
            Vt = U - W @ S
            A = np.tril(q[l, s:e] * Gam @ Kinv.T, 0 if variant != "strict_causal" else -1)
            o[l, s:e] = (q[l, s:e] * Gam) @ S + A @ Vt
            S = np.exp(G[-1])[:, None] * S + Kbar.T @ Vt
        Sout.append(S)
    return o, np.stack(Sout)


def _pins_pass(fn):
    """The oracle pins, phrased against any candidate implementation fn(q,k,v,la,beta,S0)."""
    doc = json.load(open(os.path.join(GOLDEN, "exact_small.json")))
    for c in doc["cases"]:
        arr = lambda n: np.array(c[n], dtype=np.float32)[None]
        S0 = None if c["S0"] is None else np.array(c["S0"], dtype=np.float32)[None]
        o, S = fn(arr("q"), arr("k"), arr("v"), arr("log_alpha"), np.array(c["beta"], np.float32)[None], S0)
        o_ref = np.array([[float(Fraction(x)) for x in r] for r in c["o"]])
        if np.abs(o[0] - o_ref).max() > 1e-12:
            return False
    rng = np.random.default_rng(3)
    T, d = 40, 8
    q = rng.standard_normal((1, T, d)).astype(np.float32)
    k = rng.standard_normal((1, T, d)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, d)).astype(np.float32)
    la = rng.uniform(-0.5, 0, (1, T, d)).astype(np.float32)
    beta = rng.uniform(0.1, 0.9, (1, T)).astype(np.float32)
    S0 = rng.standard_normal((1, d, d)).astype(np.float32)
    o_ref, S_ref = native.kda_fwd(q, k, v, la, beta, S0)
    o, S = fn(q, k, v, la, beta, S0)
    return np.abs(o - o_ref).max() < 1e-10 and np.abs(S - S_ref).max() < 1e-10


def test_real_recurrence_passes_its_pins():
    assert _pins_pass(lambda *a: _loop(*a, variant="none"))
    assert _pins_pass(lambda *a: _chunk_mutant(*a[:5], a[5] if a[5] is not None else np.zeros((1, a[1].shape[2], a[2].shape[2]), np.float32), variant="none"))


def test_every_recurrence_mutant_fails_a_pin():
    for variant in ("predict_undecayed", "read_before_write", "decay_after_write", "no_beta_in_erase",
                    "transposed_read"):
        assert not _pins_pass(lambda *a, _v=variant: _loop(*a, variant=_v)), variant


def test_every_chunk_mutant_fails_a_pin():
    z = lambda a: a[5] if a[5] is not None else np.zeros((1, a[1].shape[2], a[2].shape[2]), np.float32)
    for variant in ("kbar_forward_decay", "akk_with_diag", "strict_causal"):
        assert not _pins_pass(lambda *a, _v=variant: _chunk_mutant(*a[:5], z(a), variant=_v)), variant
