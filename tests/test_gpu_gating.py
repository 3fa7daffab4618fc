"""GPU parity of the fused prologue g = g_min * Sigmoid(e^{A_h} z) and epilogue
Sigmoid(gate) * RMSNorm(o) around the KDA core (section 2.2 of the Kimi K3 reading notes: decay
lower-bound equation, output gate equation), in prefill (kda_chunk_fwd_varlen) and decode
(kda_decode_step_gated), against the fp64 oracle: oracle.gating for the elementwise steps, the
token-loop oracle for the core.

Tolerances: o and the state as everywhere (max-abs 2e-2, rel-L2 1e-2). The gated output
y = s w o / r(o), r(o) = sqrt(mean(o^2) + eps), moves by |dy| <= 2 |s w| max|do| / r(o) for an
error do in o (the derivative of o / r(o) has norm <= 2 / r(o)), plus its own rounding to the
output type; each token is held to that bound with max|do| = 2e-2.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_78_amd as kda
from gated_delta_rule_78_amd import synth
from oracle import gating, native
from tests.parity import TOL_O, TOL_S, assert_close, host32, rel_l2_per_lane, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
BF16, F32 = torch.bfloat16, torch.float32
G_MIN, EPS = -5.0, 1e-6


def check_gated(tag, y, o_ref, gate, w, odt):
    """y (device) against the oracle epilogue of o_ref, token by token within the derived bound."""
    g = host32(gate).astype(np.float64)
    wv = host32(w).astype(np.float64)
    y_ref = gating.gated_rmsnorm(o_ref, g, wv, EPS)
    r = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + EPS)
    rnd = 2.0 ** -8 if odt == BF16 else 1e-6
    bound = 2.0 * gating.sigmoid(g) * np.abs(wv) * TOL_O[BF16] / r + rnd * np.abs(y_ref) + 1e-6
    err = np.abs(host32(y).astype(np.float64) - y_ref)
    worst = float(np.max(err / bound))
    say("%s: max|y - y_ref| = %.3e, worst error / bound = %.3f" % (tag, float(err.max()), worst))
    assert worst <= 1.0


def packed_case(lens, H, d, seed, s0_std=0.3):
    q, k, v, la, beta, cu, S0 = synth.packed_inputs(lens, H, d, d, BF16, device=DEV, seed_base=seed, s0_std=s0_std)
    T = int(cu[-1])
    z, A_log, gate, w = synth.gating_inputs((H, T), H, d, d, BF16, device=DEV, seed=seed + 1)
    return q, k, v, la, beta, cu, S0, z, A_log, gate, w


def oracle_packed(q, k, v, la_or_g, beta, cu, S0, E):
    return native.kda_varlen(host32(q), host32(k), host32(v), la_or_g, host32(beta), cu.cpu().numpy(),
                             None if S0 is None else host32(S0), ckpt_every=E)


@pytest.mark.parametrize("segments", [0, 3])
def test_prologue_packed(segments):
    """Decay from z: log_alpha is not passed at all."""
    lens = [700, 0, 333, 1029, 64]
    H, d, E = 4, 128, 256
    q, k, v, la, beta, cu, S0, z, A_log, gate, w = packed_case(lens, H, d, 6100 + segments)
    say("prologue packed: lens=%s H=%d segments=%d" % (lens, H, segments))
    o, S_T, ck, offs = kda.chunk_fwd_varlen(q, k, v, None, beta, cu, S0, ckpt_every=E, segments=segments,
                                            z=z, A_log=A_log, g_min=G_MIN)
    torch.cuda.synchronize()
    g = gating.log_decay(host32(z), host32(A_log)[:, None, None], G_MIN)
    ref = oracle_packed(q, k, v, g.astype(np.float32), beta, cu, S0, E)
    N = len(lens)
    assert_close("prologue packed", BF16, host32(o), ref[0], host32(S_T).reshape(N * H, d, d), ref[1].reshape(N * H, d, d))
    n = int(ref[3][-1])
    es = rel_l2_per_lane(host32(ck[:n]).reshape(n * H, -1), ref[2].reshape(n * H, -1))
    say("prologue packed: checkpoints relL2 = %.3e" % es)
    assert np.array_equal(offs.cpu().numpy(), ref[3]) and es <= TOL_S[BF16]


@pytest.mark.parametrize("odt", [BF16, F32])
def test_epilogue_packed(odt):
    lens = [513, 1, 900, 66]
    H, d = 3, 128
    q, k, v, la, beta, cu, S0, z, A_log, gate, w = packed_case(lens, H, d, 6200)
    say("epilogue packed: lens=%s H=%d out=%s" % (lens, H, odt))
    y, S_T, _, _ = kda.chunk_fwd_varlen(q, k, v, la, beta, cu, S0, out_dtype=odt, gate=gate, norm_weight=w, eps=EPS)
    torch.cuda.synchronize()
    ref = oracle_packed(q, k, v, host32(la), beta, cu, S0, 0)
    N = len(lens)
    es = rel_l2_per_lane(host32(S_T).reshape(N * H, -1), ref[1].reshape(N * H, -1))
    assert es <= TOL_S[BF16]
    check_gated("epilogue packed", y, ref[0], gate, w, odt)


def test_prologue_and_epilogue_equal_lengths():
    """Both fused steps, equal-length layout [N,H,T,d], d = 64, no norm weight (ones)."""
    N, H, T, d = 2, 3, 64 * 5 + 9, 64
    q, k, v, la, beta, S0 = synth.prefill_inputs(N, H, T, d, d, BF16, device=DEV, seed_base=6300, s0_std=0.2)
    z, A_log, gate, _ = synth.gating_inputs((N, H, T), H, d, d, BF16, device=DEV, seed=6301)
    say("both fused, equal lengths: N=%d H=%d T=%d d=%d" % (N, H, T, d))
    y, S_T, _, _ = kda.chunk_fwd_varlen(q, k, v, None, beta, None, S0, z=z, A_log=A_log, g_min=G_MIN, gate=gate,
                                        eps=EPS)
    torch.cuda.synchronize()
    g = gating.log_decay(host32(z), host32(A_log)[None, :, None, None], G_MIN).astype(np.float32)
    f = lambda x: host32(x).reshape((N * H,) + tuple(x.shape[2:]))
    o_ref, S_ref = native.kda_fwd(f(q), f(k), f(v), g.reshape(N * H, T, d), f(beta), f(S0))
    es = rel_l2_per_lane(host32(S_T).reshape(N * H, -1), S_ref.reshape(N * H, -1))
    assert es <= TOL_S[BF16]
    check_gated("both fused", y.reshape(N * H, T, d), o_ref, gate.reshape(N * H, T, d), torch.ones(d), BF16)


@pytest.mark.parametrize("dt", [BF16, F32])
def test_decode_gated(dt):
    N, H, d = 64, 8, 128
    S = synth.decode_state(N, H, d, d, 0.3, device=DEV, seed=6400)
    q, k, v, la, beta = synth.decode_tokens(N, H, d, d, dt, device=DEV, seed=6401)
    z, A_log, gate, w = synth.gating_inputs((N, H), H, d, d, dt, device=DEV, seed=6402)
    S_host = host32(S)
    say("decode gated: N=%d H=%d d=%d in=%s" % (N, H, d, dt))
    y = kda.decode_step(q, k, v, None, beta, S, z=z, A_log=A_log, g_min=G_MIN, gate=gate, norm_weight=w, eps=EPS)
    torch.cuda.synchronize()
    g = gating.log_decay(host32(z), host32(A_log)[None, :, None], G_MIN).astype(np.float32)
    f = lambda x: host32(x).reshape((N * H,) + tuple(x.shape[2:]))
    o_ref, S_ref = native.kda_decode(f(q), f(k), f(v), g.reshape(N * H, d), f(beta), S_host.reshape(N * H, d, d))
    es = rel_l2_per_lane(host32(S).reshape(N * H, -1), S_ref.reshape(N * H, -1))
    say("decode gated: relL2(S) = %.3e" % es)
    assert es <= TOL_S[dt]
    check_gated("decode gated", y.reshape(N * H, d), o_ref, gate.reshape(N * H, d), w, dt)
