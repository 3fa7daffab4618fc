"""Invariants the pages fix, checked on the HIP path (prefill through kda_chunk_fwd, decode through
kda_decode_step), each against both the fp64 oracle and a closed form:

- the overwrite example of the Kimi K3 CSDN mirror, section 2.1 ("KDA 改变了什么"): with no decay
  and a full write (alpha = 1, beta = 1), orthonormal keys and a zero start, a later write to the
  same key replaces the earlier value instead of adding to it, so the state maps every key to the
  value it was written last, and a query with that key reads it back;
- unit-key recall (Kimi K3 reading notes, section 2.2, state recurrence equation): with beta = 1
  and a key of unit norm, (I - k k^T) k = 0, so S_t^T k_t = v_t after the write for any decay; a
  query equal to the key therefore returns v_t exactly;
- linearity: for fixed q, k, alpha, beta the recurrence is linear in (V, S0) jointly.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_78_amd as kda
from gated_delta_rule_78_amd import synth
from oracle import native
from tests.parity import TOL_O, TOL_S, host32, max_abs, rel_l2_per_lane, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
BF16, F32 = torch.bfloat16, torch.float32


def token(x, t):
    """Token t of every lane of a [1, L, T, ...] prefill tensor as a decode input [L, 1, ...]."""
    return x[0, :, t, None].contiguous()


def overwrite_sequence(T, d, shift):
    """Key index i_t (a standard basis vector of R^d: exact in bf16), written value v_t (multiples
    of 1/4 in [-2, 2]: exact in bf16) and query index (the key written at t, or another key)."""
    idx = np.array([t % d if t < d else (7 * t + shift) % d for t in range(T)])
    v = np.array([[((t * 31 + j * 7 + shift) % 17 - 8) / 4.0 for j in range(d)] for t in range(T)])
    qidx = np.array([idx[t] if t % 3 else (idx[t] + 5 + shift) % d for t in range(T)])
    return idx, v, qidx


def overwrite_closed_form(idx, v, qidx, d):
    """Last-write table: o_t = the value last written to key qidx[t] up to and including t (zero if
    never written), S_T[i] = the value last written to key i."""
    T = len(idx)
    table = np.zeros((d, v.shape[1]))
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        table[idx[t]] = v[t]
        o[t] = table[qidx[t]]
    return o, table


def test_overwrite_example_prefill_and_decode():
    d, T, lanes = 128, 64 * 4 + 37, 2
    eye = np.eye(d)
    qs, ks, vs, refs = [], [], [], []
    for lane in range(lanes):
        idx, v, qidx = overwrite_sequence(T, d, shift=lane)
        qs.append(eye[qidx]); ks.append(eye[idx]); vs.append(v)
        refs.append(overwrite_closed_form(idx, v, qidx, d))
    q = torch.tensor(np.stack(qs)[None], dtype=BF16, device=DEV)
    k = torch.tensor(np.stack(ks)[None], dtype=BF16, device=DEV)
    v = torch.tensor(np.stack(vs)[None], dtype=BF16, device=DEV)
    la = torch.zeros(1, lanes, T, d, dtype=BF16, device=DEV)           # alpha = 1
    beta = torch.ones(1, lanes, T, dtype=BF16, device=DEV)             # full write
    say("overwrite example: d=%d T=%d lanes=%d (prefill, decode)" % (d, T, lanes))
    o, S_T = kda.chunk_fwd(q, k, v, la, beta, None, out_dtype=F32)
    # decode: the same tokens one step at a time from the zero state
    S = torch.zeros(lanes, 1, d, d, dtype=F32, device=DEV)
    od = torch.stack([kda.decode_step(*(token(x, t) for x in (q, k, v, la, beta)), S, out_dtype=F32)[:, 0]
                      for t in range(T)], dim=1)
    torch.cuda.synchronize()
    f = lambda x: host32(x).reshape((lanes,) + tuple(x.shape[2:]))
    o_ref, S_ref = native.kda_fwd(f(q), f(k), f(v), f(la), host32(beta).reshape(lanes, T))
    for lane in range(lanes):
        o_cf, S_cf = refs[lane]
        assert np.array_equal(o_ref[lane], o_cf) and np.array_equal(S_ref[lane], S_cf)   # the oracle is exact here
    e_pre = max_abs(host32(o)[0], o_ref)
    e_dec = max_abs(host32(od), o_ref)
    e_S = max(max_abs(host32(S_T)[0], S_ref), max_abs(host32(S)[:, 0], S_ref))
    say("overwrite: prefill max|o-o_ref| %.3e, decode %.3e, states %.3e" % (e_pre, e_dec, e_S))
    assert e_pre <= TOL_O[BF16] and e_dec <= TOL_O[BF16] and e_S <= TOL_O[BF16]


def unit_keys(L, T, d, gen):
    """Keys with exactly unit norm in bf16: +-1/8 on 64 random channels (64 / 64 = 1)."""
    k = torch.zeros(L, T, d)
    for lane in range(L):
        for t in range(T):
            ch = torch.randperm(d, generator=gen)[:64]
            k[lane, t, ch] = (torch.randint(0, 2, (64,), generator=gen).float() * 2 - 1) / 8.0
    return k


@pytest.mark.parametrize("la_range", [(-0.5, -0.001), (-5.0, 0.0)])
def test_unit_key_recall_prefill_and_decode(la_range):
    """beta = 1, unit keys, q_t = k_t: o_t = S_t^T k_t = v_t for every token, whatever the decay."""
    d, T, L = 128, 64 * 3 + 11, 3
    gen = torch.Generator().manual_seed(9100)
    k = unit_keys(L, T, d, gen)
    assert torch.equal((k.double() ** 2).sum(-1), torch.ones(L, T, dtype=torch.float64))
    _, _, v, la, _, S0 = synth.prefill_inputs(1, L, T, d, d, BF16, seed_base=9101, s0_std=0.5, log_alpha_range=la_range)
    q = k.to(BF16)[None].to(DEV)
    kk = q.clone()
    v, la, S0 = v.to(DEV), la.to(DEV), S0.to(DEV)
    beta = torch.ones(1, L, T, dtype=BF16, device=DEV)
    say("unit-key recall: d=%d T=%d lanes=%d log_alpha=%s" % (d, T, L, la_range))
    o, S_T = kda.chunk_fwd(q, kk, v, la, beta, S0, out_dtype=F32)
    S = S0[0][:, None].clone()
    od = torch.stack([kda.decode_step(*(token(x, t) for x in (q, kk, v, la, beta)), S, out_dtype=F32)[:, 0]
                      for t in range(T)], dim=1)
    torch.cuda.synchronize()
    vv = host32(v)[0]
    e_pre, e_dec = max_abs(host32(o)[0], vv), max_abs(host32(od), vv)
    # the final state recalls the last token's value along its key
    recall = np.einsum("lcj,lc->lj", host32(S_T)[0].astype(np.float64), host32(kk)[0, :, -1].astype(np.float64))
    e_rec = max_abs(recall, vv[:, -1])
    say("unit-key recall: prefill max|o-v| %.3e, decode %.3e, S_T^T k_T vs v_T %.3e" % (e_pre, e_dec, e_rec))
    assert e_pre <= TOL_O[BF16] and e_dec <= 1e-4 and e_rec <= TOL_O[BF16]


def test_linearity_in_v_and_s0():
    """(o, S_T) of V1 + V2 from S01 + S02 equals the sum of the two runs. V1, V2 are multiples of
    1/16 in [-4, 4], so V1 + V2 is exact in bf16 and the three calls see exact inputs."""
    B, H, T, d = 1, 4, 64 * 5 + 23, 128
    q, k, v1, la, beta, S01 = synth.prefill_inputs(B, H, T, d, d, BF16, device=DEV, seed_base=9200, s0_std=0.3)
    _, _, v2, _, _, S02 = synth.prefill_inputs(B, H, T, d, d, BF16, device=DEV, seed_base=9300, s0_std=0.3)
    quant = lambda x: (torch.round(x.float() * 16).clamp(-64, 64) / 16).to(BF16)
    v1, v2 = quant(v1), quant(v2)
    v3 = (v1.float() + v2.float()).to(BF16)
    assert torch.equal(v3.float(), v1.float() + v2.float())
    say("linearity: B=%d H=%d T=%d d=%d" % (B, H, T, d))
    o1, s1 = kda.chunk_fwd(q, k, v1, la, beta, S01, out_dtype=F32)
    o2, s2 = kda.chunk_fwd(q, k, v2, la, beta, S02, out_dtype=F32)
    o3, s3 = kda.chunk_fwd(q, k, v3, la, beta, S01 + S02, out_dtype=F32)
    torch.cuda.synchronize()
    e_o = max_abs(host32(o3), host32(o1) + host32(o2))
    e_s = rel_l2_per_lane(host32(s3).reshape(H, -1), (host32(s1) + host32(s2)).reshape(H, -1))
    f = lambda x: host32(x).reshape((H,) + tuple(x.shape[2:]))
    o_ref, S_ref = native.kda_fwd(f(q), f(k), f(v3), f(la), host32(beta).reshape(H, T), f(S01 + S02))
    say("linearity: max|o(V1+V2) - o(V1) - o(V2)| %.3e relL2(S) %.3e; max|o(V1+V2) - oracle| %.3e"
        % (e_o, e_s, max_abs(host32(o3)[0], o_ref)))
    assert e_o <= TOL_O[BF16] and e_s <= TOL_S[BF16]
    assert max_abs(host32(o3)[0], o_ref) <= TOL_O[BF16]
