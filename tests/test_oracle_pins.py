"""Pins of the oracle to facts fixed by the pages and by mathematics (CPU only).

The recurrence under test is the KDA state equation of section 2.2 of the Kimi K3 reading notes
(liuzhao09.github.io/papers/kimi-k3.html); the chunk form is that section's chunk equations;
the affine pair and split/resume come from section 2.5 and its Figure 12.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import chunked, exact, native, recurrence

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
RNG = np.random.default_rng(12345)


def _rand_inputs(L, T, dk, dv, la_lo=-0.5, la_hi=-0.001, rng=RNG, s0=True):
    """Small fp32 inputs shaped like the workloads (unit-norm q, k)."""
    q = rng.standard_normal((L, T, dk)).astype(np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((L, T, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((L, T, dv)).astype(np.float32)
    la = rng.uniform(la_lo, la_hi, (L, T, dk)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((L, T))))).astype(np.float32)
    S0 = (0.3 * rng.standard_normal((L, dk, dv))).astype(np.float32) if s0 else None
    return q, k, v, la, beta, S0


def _frac(x):
    return Fraction(x)


# ---- 1. exact rational brute force (stored fixture written from oracle.exact) ----

def test_golden_exact_rationals_match_c_and_numpy():
    doc = json.load(open(os.path.join(GOLDEN, "exact_small.json")))
    assert doc["citation"]
    for c in doc["cases"]:
        q, k, v, la = (np.array(c[n], dtype=np.float32)[None] for n in ("q", "k", "v", "log_alpha"))
        beta = np.array(c["beta"], dtype=np.float32)[None]
        S0 = None if c["S0"] is None else np.array(c["S0"], dtype=np.float32)[None]
        o_ref = np.array([[float(Fraction(x)) for x in row] for row in c["o"]])
        S_ref = np.array([[float(Fraction(x)) for x in row] for row in c["S_T"]])
        o_c, S_c = native.kda_fwd(q, k, v, la, beta, S0)
        o_n, S_n = recurrence.kda_fwd(q, k, v, la, beta, S0)
        for o, S in ((o_c, S_c), (o_n, S_n)):
            assert np.abs(o[0] - o_ref).max() < 1e-12
            assert np.abs(S[0] - S_ref).max() < 1e-12


def test_exact_bruteforce_fresh_cases():
    """Exact arithmetic vs both fp64 loops on fresh random dyadic inputs (d=2..4, T<=16)."""
    rng = np.random.default_rng(7)
    for dk, dv, T in ((2, 3, 5), (4, 2, 16), (3, 3, 11)):
        q = (rng.integers(-8, 9, (T, dk)) / 8).astype(np.float32)
        k = (rng.integers(-8, 9, (T, dk)) / 8).astype(np.float32)
        v = (rng.integers(-16, 17, (T, dv)) / 8).astype(np.float32)
        beta = (rng.integers(1, 16, T) / 16).astype(np.float32)
        la = rng.uniform(-0.6, 0.0, (T, dk)).astype(np.float32)
        S0 = (rng.integers(-16, 17, (dk, dv)) / 16).astype(np.float32)
        alpha = [[Fraction(float(np.exp(np.float64(x)))) for x in row] for row in la]
        fr = lambda m: [[_frac(float(x)) for x in row] for row in m]
        o_x, S_x = exact.kda_fwd(fr(q), fr(k), fr(v), alpha, [_frac(float(b)) for b in beta], fr(S0))
        o_x = np.array([[float(x) for x in r] for r in o_x])
        S_x = np.array([[float(x) for x in r] for r in S_x])
        o_c, S_c = native.kda_fwd(q[None], k[None], v[None], la[None], beta[None], S0[None])
        assert np.abs(o_c[0] - o_x).max() < 1e-12 and np.abs(S_c[0] - S_x).max() < 1e-12


# ---- 2. the C loop, the numpy loop and the explicit product form agree ----

def test_c_numpy_product_form_agree():
    q, k, v, la, beta, S0 = _rand_inputs(3, 40, 8, 6)
    o_c, S_c = native.kda_fwd(q, k, v, la, beta, S0)
    o_n, S_n = recurrence.kda_fwd(q, k, v, la, beta, S0)
    assert np.abs(o_c - o_n).max() < 1e-13 and np.abs(S_c - S_n).max() < 1e-13
    for l in range(3):
        o_p, S_p = recurrence.kda_product_form(q[l], k[l], v[l], la[l], beta[l], S0[l])
        assert np.abs(o_p - o_c[l]).max() < 1e-12 and np.abs(S_p - S_c[l]).max() < 1e-12


def test_c_oracle_row_selection_and_threads():
    q, k, v, la, beta, S0 = _rand_inputs(2, 50, 8, 40)      # 40 columns: three column blocks
    o, S = native.kda_fwd(q, k, v, la, beta, S0, threads=1)
    rows = [0, 3, 17, 49]
    o_r, S_r = native.kda_fwd(q, k, v, la, beta, S0, rows=rows, threads=4)
    assert np.array_equal(o_r, o[:, rows]) and np.array_equal(S_r, S)
    with pytest.raises(ValueError):
        native.kda_fwd(q, k, v, la, beta, S0, rows=[3, 3])


# ---- 3. chunked form == recurrence (pins the derived U, W and chunk-end state) ----

@pytest.mark.parametrize("C", [1, 7, 16, 64, 130])
def test_chunked_equals_recurrence(C):
    q, k, v, la, beta, S0 = _rand_inputs(2, 130, 16, 12)
    o_r, S_r = native.kda_fwd(q, k, v, la, beta, S0)
    o_k, S_k = chunked.kda_chunked(q, k, v, la, beta, S0, C=C)
    assert np.abs(o_k - o_r).max() < 1e-12 and np.abs(S_k - S_r).max() < 1e-12


def test_chunked_full_decay_domain_fp64():
    """log alpha down to the lower bound -5 (decay-bound equation): fine in fp64 at C=64."""
    q, k, v, la, beta, S0 = _rand_inputs(1, 100, 8, 8, la_lo=-5.0, la_hi=0.0)
    o_r, S_r = native.kda_fwd(q, k, v, la, beta, S0)
    o_k, S_k = chunked.kda_chunked(q, k, v, la, beta, S0, C=64)
    assert np.abs(o_k - o_r).max() < 1e-10 and np.abs(S_k - S_r).max() < 1e-10


# ---- 4. special cases with closed forms ----

def test_alpha1_beta0_is_identity():
    """alpha = 1, beta = 0: the state never changes and o_t = S0^T q_t (a plain matmul)."""
    q, k, v, la, beta, S0 = _rand_inputs(2, 20, 8, 5)
    la[:] = 0.0
    beta[:] = 0.0
    o, S = native.kda_fwd(q, k, v, la, beta, S0)
    assert np.array_equal(S, S0.astype(np.float64))
    assert np.abs(o - np.matmul(q.astype(np.float64), S0.astype(np.float64))).max() < 1e-14


def test_beta0_closed_form_decay():
    """beta = 0: S_t = Diag(gamma^{1->t}) S0 and o_t = S0^T (gamma^{1->t} * q_t)."""
    q, k, v, la, beta, S0 = _rand_inputs(1, 30, 6, 4)
    beta[:] = 0.0
    o, S = native.kda_fwd(q, k, v, la, beta, S0)
    gam = np.exp(np.cumsum(la[0].astype(np.float64), axis=0))        # [T, dk]
    o_cf = (gam * q[0]) @ S0[0].astype(np.float64)
    S_cf = gam[-1][:, None] * S0[0]
    assert np.abs(o[0] - o_cf).max() < 1e-13 and np.abs(S[0] - S_cf).max() < 1e-13


def test_beta0_closed_form_full_decay_domain():
    """beta = 0 over the whole decay domain log alpha in [-5, 0] (decay lower-bound equation):
    the closed form of the test above, with cumulative decays down to about -300."""
    q, k, v, la, beta, S0 = _rand_inputs(1, 130, 6, 4, la_lo=-5.0, la_hi=0.0)
    beta[:] = 0.0
    o, S = native.kda_fwd(q, k, v, la, beta, S0)
    gam = np.exp(np.cumsum(la[0].astype(np.float64), axis=0))
    o_cf = (gam * q[0]) @ S0[0].astype(np.float64)
    S_cf = gam[-1][:, None] * S0[0]
    assert np.abs(o[0] - o_cf).max() < 1e-13 and np.abs(S[0] - S_cf).max() < 1e-13


def test_beta1_unit_key_recall():
    """beta = 1 and ||k|| = 1: after the write S_t^T k_t = v_t, whatever alpha and the old state;
    reading with q_t = k_t therefore returns v_t exactly (up to rounding)."""
    q, k, v, la, beta, S0 = _rand_inputs(2, 25, 8, 6, la_lo=-5.0, la_hi=0.0)
    k64 = k.astype(np.float64)
    k = (k64 / np.linalg.norm(k64, axis=-1, keepdims=True)).astype(np.float32)
    beta[:] = 1.0
    o, _ = native.kda_fwd(k, k, v, la, beta, S0)
    err = np.abs(o - v).max()
    # ||k||^2 is 1 only up to fp32 rounding of k's entries
    assert err < 1e-5


def test_overwrite_worked_example():
    doc = json.load(open(os.path.join(GOLDEN, "overwrite_example.json")))
    arr = lambda n: np.array(doc[n], dtype=np.float32)[None]
    o, S = native.kda_fwd(arr("q"), arr("k"), arr("v"), arr("log_alpha"), arr("beta")[0][None])
    assert np.array_equal(o[0], np.array(doc["expected_o"], dtype=np.float64))
    assert np.array_equal(S[0], np.array(doc["expected_S_T"], dtype=np.float64))
    # a plain additive (non-delta) memory would report the sum of both dates
    k = arr("k")[0].astype(np.float64)
    v = arr("v")[0].astype(np.float64)
    assert (k.T @ v)[0, 0] == doc["stacking_o_last"]


# ---- 5. structure: linearity, affine pair, split/resume, decode, norm bound ----

def test_linearity_in_v_and_s0():
    q, k, v, la, beta, S0 = _rand_inputs(1, 33, 6, 5)
    _, _, v2, _, _, S02 = _rand_inputs(1, 33, 6, 5)
    a, b = 0.75, -1.25
    o1, S1 = recurrence.kda_fwd(q, k, v, la, beta, S0)
    o2, S2 = recurrence.kda_fwd(q, k, v2, la, beta, S02)
    f64 = lambda x: x.astype(np.float64)
    o3, S3 = recurrence.kda_fwd(q, k, a * f64(v) + b * f64(v2), la, beta, a * f64(S0) + b * f64(S02))
    assert np.abs(o3 - (a * o1 + b * o2)).max() < 1e-12 and np.abs(S3 - (a * S1 + b * S2)).max() < 1e-12


def test_affine_pair_matches_transition_product():
    """Section 2.5: S_out = S~ + M S_in. M must equal the product of the per-token transition
    matrices, and S~ the output state from a zero entry state."""
    q, k, v, la, beta, S0 = _rand_inputs(1, 150, 8, 5)
    M, St = chunked.segment_affine_pair(k[0], v[0], la[0], beta[0], C=64)
    P = np.eye(8)
    for t in range(150):
        P = recurrence.transition(k[0, t], la[0, t], beta[0, t]) @ P
    _, S_zero = native.kda_fwd(q, k, v, la, beta, None)
    _, S_full = native.kda_fwd(q, k, v, la, beta, S0)
    assert np.abs(M - P).max() < 1e-12
    assert np.abs(St - S_zero[0]).max() < 1e-12
    assert np.abs(S_full[0] - (St + M @ S0[0])).max() < 1e-12


def test_segment_composition_gives_exact_entry_states():
    q, k, v, la, beta, S0 = _rand_inputs(1, 300, 8, 4, la_lo=-0.02, la_hi=0.0)
    bounds = [0, 64, 150, 300]
    pairs = [chunked.segment_affine_pair(k[0, a:b], v[0, a:b], la[0, a:b], beta[0, a:b]) for a, b in
             zip(bounds[:-1], bounds[1:])]
    entries, exit_state = chunked.compose_entry_states(pairs, S0[0])
    for a, e in zip(bounds[:-1], entries):
        _, S_a = native.kda_fwd(q[:, :a], k[:, :a], v[:, :a], la[:, :a], beta[:, :a], S0) if a else (None, S0[None])
        assert np.abs(np.asarray(S_a).reshape(e.shape) - e).max() < 1e-11
    _, S_T = native.kda_fwd(q, k, v, la, beta, S0)
    assert np.abs(S_T[0] - exit_state).max() < 1e-11


def test_split_resume_at_boundary():
    """Figure 12: restore the state at a hit boundary B and continue, instead of recomputing."""
    q, k, v, la, beta, S0 = _rand_inputs(1, 300, 8, 8)
    B = 256
    o_full, S_full = native.kda_fwd(q, k, v, la, beta, S0)
    o_a, S_B = native.kda_fwd(q[:, :B], k[:, :B], v[:, :B], la[:, :B], beta[:, :B], S0)
    o_b, S_end = native.kda_fwd(q[:, B:], k[:, B:], v[:, B:], la[:, B:], beta[:, B:], S_B.astype(np.float32))
    # resuming from an fp32 copy of the state: agreement to fp32 rounding of S_B
    assert np.abs(o_a - o_full[:, :B]).max() == 0
    assert np.abs(o_b - o_full[:, B:]).max() < 1e-6 and np.abs(S_end - S_full).max() < 1e-6


def test_decode_step_is_one_more_token():
    q, k, v, la, beta, S0 = _rand_inputs(3, 21, 8, 8)
    o_full, S_full = native.kda_fwd(q, k, v, la, beta, S0)
    _, S_pre = native.kda_fwd(q[:, :20], k[:, :20], v[:, :20], la[:, :20], beta[:, :20], S0)
    o_d, S_d = native.kda_decode(q[:, 20], k[:, 20], v[:, 20], la[:, 20], beta[:, 20], S_pre.astype(np.float32))
    assert np.abs(o_d - o_full[:, 20]).max() < 1e-6 and np.abs(S_d - S_full).max() < 1e-6


def test_state_norm_bound():
    """With ||k||=1 and beta in [0,1], ||(I - beta k k^T) Diag(alpha)||_2 <= 1, so
    ||S_t||_2 <= ||S_{t-1}||_2 + beta_t ||v_t||."""
    q, k, v, la, beta, S0 = _rand_inputs(1, 60, 6, 6, la_lo=-0.05, la_hi=0.0)
    S = S0.astype(np.float64)
    for t in range(60):
        _, S_next = native.kda_fwd(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], la[:, t:t + 1], beta[:, t:t + 1],
                                   S.astype(np.float32))
        bound = np.linalg.norm(S.astype(np.float32).astype(np.float64)[0], 2) + beta[0, t] * np.linalg.norm(v[0, t])
        assert np.linalg.norm(S_next[0], 2) <= bound + 1e-9
        S = S_next


def test_empty_sequence_returns_entry_state():
    q, k, v, la, beta, S0 = _rand_inputs(2, 0, 4, 4)
    o, S = native.kda_fwd(q, k, v, la, beta, S0)
    assert o.shape == (2, 0, 4) and np.array_equal(S, S0.astype(np.float64))
