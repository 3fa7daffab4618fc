"""GPU parity of kda_decode_step against the fp64 oracle (one token of the recurrence of
section 2.2 of the Kimi K3 reading notes). Calls go through the C ABI via the binding."""
import numpy as np
import pytest
import torch

import gated_delta_rule_78_amd as kda
from gated_delta_rule_78_amd import synth
from oracle import native
from tests.parity import TOL_O, TOL_S, assert_close, host32, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def _flat(x):
    a = host32(x)
    return a.reshape((-1,) + a.shape[2:])


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("dt,odt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                    (torch.bfloat16, torch.float32)])
def test_decode_small(dk, dv, dt, odt):
    say("decode small dk=%d dv=%d in=%s out=%s" % (dk, dv, dt, odt))
    N, H = 5, 3
    S = synth.decode_state(N, H, dk, dv, 0.02, device=DEV, seed=11)
    S_in = host32(S).reshape(N * H, dk, dv)
    q, k, v, la, beta = synth.decode_tokens(N, H, dk, dv, dt, device=DEV, seed=12)
    o = kda.decode_step(q, k, v, la, beta, S, out_dtype=odt)
    torch.cuda.synchronize()
    o_ref, S_ref = native.kda_decode(_flat(q), _flat(k), _flat(v), _flat(la), host32(beta).reshape(-1), S_in)
    assert_close("decode", dt, host32(o).reshape(N * H, dv), o_ref, host32(S).reshape(N * H, dk, dv), S_ref)


def test_decode_chain_full_size_sampled():
    """256 sequences x 32 heads, d = 128, bf16 tokens, fp32 state; 1000 chained steps (the
    benchmark's chain), every output and the final state checked on 8 sampled (n, h) slices."""
    w = synth.DECODE_BF16_256x32
    N, H, d = w.N, w.H, w.d
    steps = 1000
    say("decode chain N=%d H=%d d=%d steps=%d" % (N, H, d, steps))
    S = synth.decode_state(N, H, d, d, w.s_std, device=DEV, seed=21)
    lanes = [0, 1, 777, 2048, 4095, 5000, 8000, N * H - 1]
    S_cur = host32(S).reshape(N * H, d, d)[lanes]
    worst_o = 0.0
    for step in range(steps):
        q, k, v, la, beta = synth.decode_tokens(N, H, d, d, w.dtype, device=DEV, seed=100 + step)
        o = kda.decode_step(q, k, v, la, beta, S)
        o_ref, S_cur = native.kda_decode(_flat(q)[lanes], _flat(k)[lanes], _flat(v)[lanes], _flat(la)[lanes],
                                         host32(beta).reshape(-1)[lanes], S_cur.astype(np.float32))
        worst_o = max(worst_o, float(np.abs(host32(o).reshape(N * H, d)[lanes] - o_ref).max()))
    torch.cuda.synchronize()
    S_gpu = host32(S).reshape(N * H, d, d)[lanes]
    assert_close("decode chain (worst step)", torch.bfloat16, np.zeros(1), np.full(1, worst_o), S_gpu, S_cur)
    assert worst_o <= TOL_O[torch.bfloat16]


def test_decode_after_prefill_is_next_token():
    """Prefill T tokens, then one decode step == prefill of T+1 tokens (last output, final state)."""
    B, H, T, d = 1, 4, 300, 128
    say("decode after prefill T=%d" % T)
    q, k, v, la, beta, _ = synth.prefill_inputs(B, H, T + 1, d, d, torch.bfloat16, device=DEV, seed_base=31)
    o_all, S_all = kda.chunk_fwd(q, k, v, la, beta, out_dtype=torch.float32)
    _, S_T = kda.chunk_fwd(q[:, :, :T].contiguous(), k[:, :, :T].contiguous(), v[:, :, :T].contiguous(),
                           la[:, :, :T].contiguous(), beta[:, :, :T].contiguous(), out_dtype=torch.float32)
    tok = lambda x: x[0, :, T].contiguous().unsqueeze(0)
    o_dec = kda.decode_step(tok(q), tok(k), tok(v), tok(la), beta[:, :, T].contiguous(), S_T,
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.abs(host32(o_dec)[0] - host32(o_all)[0, :, T]).max() <= TOL_O[torch.bfloat16]
    num = np.linalg.norm((host32(S_T) - host32(S_all)).reshape(H, -1), axis=1)
    den = np.linalg.norm(host32(S_all).reshape(H, -1), axis=1)
    assert (num / den).max() <= TOL_S[torch.bfloat16]


def test_decode_is_deterministic():
    N, H, d = 16, 4, 128
    S1 = synth.decode_state(N, H, d, d, 0.02, device=DEV, seed=41)
    S2 = S1.clone()
    q, k, v, la, beta = synth.decode_tokens(N, H, d, d, torch.bfloat16, device=DEV, seed=42)
    o1 = kda.decode_step(q, k, v, la, beta, S1)
    o2 = kda.decode_step(q, k, v, la, beta, S2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
