"""Pins of the oracle's checkpoint and packed-batch functions (CPU only).

Section 2.5 of the Kimi K3 reading notes (liuzhao09.github.io/papers/kimi-k3.html) and its
Figure 12: a prefix cache keeps KDA checkpoints only at hash-queryable endpoints (512-token hash
blocks inside 6144-token physical blocks); a hit restores the checkpoint and continues prefill.
A checkpoint is therefore the state of section 2.2's recurrence after a whole number of
checkpoint intervals, and every sequence of a batch is an independent recurrence. The pins
compare against exact rational arithmetic on tiny inputs, and plant the plausible slips
(state carried across a sequence boundary, a checkpoint one token off, inclusive offsets) to
show the pins catch them.
"""
from fractions import Fraction

import numpy as np

from oracle import exact, native

RNG = np.random.default_rng(2024)


def _dyadic(H, T, dk, dv, rng=RNG):
    q = (rng.integers(-8, 9, (H, T, dk)) / 8).astype(np.float32)
    k = (rng.integers(-8, 9, (H, T, dk)) / 8).astype(np.float32)
    v = (rng.integers(-16, 17, (H, T, dv)) / 8).astype(np.float32)
    beta = (rng.integers(1, 16, (H, T)) / 16).astype(np.float32)
    la = rng.uniform(-0.6, 0.0, (H, T, dk)).astype(np.float32)
    return q, k, v, la, beta


def _exact_lane(q, k, v, la, beta, S0):
    """Exact rational recurrence of one lane (alpha = the fp64 value of exp(la), as a Fraction)."""
    if len(q) == 0:
        return np.zeros((0, v.shape[1])), np.asarray(S0, dtype=np.float64)
    fr = lambda m: [[Fraction(float(x)) for x in row] for row in m]
    alpha = [[Fraction(float(np.exp(np.float64(x)))) for x in row] for row in la]
    o, S = exact.kda_fwd(fr(q), fr(k), fr(v), alpha, [Fraction(float(b)) for b in beta],
                         None if S0 is None else fr(S0))
    to = lambda m: np.array([[float(x) for x in r] for r in m], dtype=np.float64)
    return (to(o) if len(o) else np.zeros((0, v.shape[1]))), to(S)


def test_checkpoints_are_exact_prefix_states():
    H, T, dk, dv, E = 2, 12, 3, 2, 4
    q, k, v, la, beta = _dyadic(H, T, dk, dv)
    S0 = (RNG.integers(-16, 17, (H, dk, dv)) / 16).astype(np.float32)
    o, ST, ck = native.kda_fwd(q, k, v, la, beta, S0, ckpt_every=E)
    assert ck.shape == (H, T // E, dk, dv)
    for h in range(H):
        for j in range(1, T // E + 1):
            _, S_j = _exact_lane(q[h, :j * E], k[h, :j * E], v[h, :j * E], la[h, :j * E], beta[h, :j * E], S0[h])
            assert np.abs(ck[h, j - 1] - S_j).max() < 1e-12
    # the last checkpoint of a sequence whose length is a multiple of E is its final state
    assert np.array_equal(ck[:, -1], ST)


def _packed_case():
    lens = [5, 0, 7, 4, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    H, dk, dv = 2, 3, 2
    T = int(cu[-1])
    q, k, v, la, beta = _dyadic(H, T, dk, dv)
    S0 = (RNG.integers(-16, 17, (len(lens), H, dk, dv)) / 16).astype(np.float32)
    return lens, cu, q, k, v, la, beta, S0


def _check_packed(fn, E=4):
    """The pins of a packed-batch function fn(q,k,v,la,beta,cu,S0,E) -> (o, S_T, ck, offs):
    per (sequence, head) exact outputs, final states and checkpoints, and the offsets."""
    lens, cu, q, k, v, la, beta, S0 = _packed_case()
    o, ST, ck, offs = fn(q, k, v, la, beta, cu, S0, E)
    exp_offs = np.concatenate([[0], np.cumsum([n // E for n in lens])])
    if not np.array_equal(np.asarray(offs), exp_offs) or ck.shape[0] != exp_offs[-1]:
        return False
    for s, n in enumerate(lens):
        a = int(cu[s])
        for h in range(q.shape[0]):
            sl = slice(a, a + n)
            o_x, S_x = _exact_lane(q[h, sl], k[h, sl], v[h, sl], la[h, sl], beta[h, sl], S0[s, h])
            if n and np.abs(o[h, sl] - o_x).max() >= 1e-12:
                return False
            if np.abs(ST[s, h] - S_x).max() >= 1e-12:
                return False
            for j in range(1, n // E + 1):
                _, S_j = _exact_lane(q[h, a:a + j * E], k[h, a:a + j * E], v[h, a:a + j * E], la[h, a:a + j * E],
                                     beta[h, a:a + j * E], S0[s, h])
                if np.abs(ck[offs[s] + j - 1, h] - S_j).max() >= 1e-12:
                    return False
    return True


def _real(q, k, v, la, beta, cu, S0, E):
    return native.kda_varlen(q, k, v, la, beta, cu, S0, ckpt_every=E)


def test_packed_batch_exact():
    assert _check_packed(_real)


def test_packed_batch_empty_sequence_keeps_entry_state():
    lens, cu, q, k, v, la, beta, S0 = _packed_case()
    o, ST, ck, offs = _real(q, k, v, la, beta, cu, S0, 4)
    assert lens[1] == 0 and np.array_equal(ST[1], S0[1].astype(np.float64)) and offs[2] == offs[1]


# ---- planted slips: each must fail the pins above ----

def _carried_state(q, k, v, la, beta, cu, S0, E):
    """Slip: one recurrence over the whole packed row range (state not reset at boundaries)."""
    H = q.shape[0]
    o, ST_all = native.kda_fwd(q, k, v, la, beta, S0[0])
    N = len(cu) - 1
    ST = np.zeros((N,) + ST_all.shape)
    cks, offs = [], [0]
    for s in range(N):
        b = int(cu[s + 1])
        _, ST[s] = native.kda_fwd(q[:, :b], k[:, :b], v[:, :b], la[:, :b], beta[:, :b], S0[0]) if b else (None, S0[0])
        n = (int(cu[s + 1]) - int(cu[s])) // E
        for j in range(1, n + 1):
            e = int(cu[s]) + j * E
            cks.append(native.kda_fwd(q[:, :e], k[:, :e], v[:, :e], la[:, :e], beta[:, :e], S0[0])[1])
        offs.append(offs[-1] + n)
    ck = np.stack(cks) if cks else np.zeros((0, H) + ST_all.shape[1:])
    return o, ST, ck, np.array(offs)


def _early_checkpoint(q, k, v, la, beta, cu, S0, E):
    """Slip: checkpoint j taken after j*E - 1 tokens."""
    o, ST, ck, offs = _real(q, k, v, la, beta, cu, S0, E)
    ck = ck.copy()
    for s in range(len(cu) - 1):
        a = int(cu[s])
        for j in range(1, (int(cu[s + 1]) - a) // E + 1):
            e = a + j * E - 1
            ck[offs[s] + j - 1] = native.kda_fwd(q[:, a:e], k[:, a:e], v[:, a:e], la[:, a:e], beta[:, a:e], S0[s])[1]
    return o, ST, ck, offs


def _inclusive_offsets(q, k, v, la, beta, cu, S0, E):
    """Slip: offsets[s] counts sequence s's own checkpoints."""
    o, ST, ck, offs = _real(q, k, v, la, beta, cu, S0, E)
    return o, ST, ck, np.concatenate([offs[1:], offs[-1:]])


def test_planted_slips_fail_the_pins():
    for slip in (_carried_state, _early_checkpoint, _inclusive_offsets):
        assert not _check_packed(slip), slip.__name__
