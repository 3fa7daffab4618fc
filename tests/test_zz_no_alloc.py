"""kda_chunk_fwd_noalloc (the prefill with its workspace in the library's fixed per-device scratch,
for callers that cannot allocate) against kda_chunk_fwd with a caller workspace: two calls in a row
through the C ABI, the second smaller, both checked against the allocating call bit for bit and
against the fp64 oracle to the bf16 bars."""
import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_78_amd as kda
from gated_delta_rule_78_amd import synth
from tests.parity import TOL_O, TOL_S, host32, max_abs, oracle_prefill, rel_l2_per_lane, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
BF16 = torch.bfloat16


def noalloc_call(q, k, v, la, beta, S0):
    """kda_chunk_fwd_noalloc through the C ABI with outputs the test allocates."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = torch.empty(B, H, T, dv, device=DEV, dtype=BF16)
    S_T = torch.empty(B, H, dk, dv, device=DEV, dtype=torch.float32)
    desc = kda.ChunkDesc(B, H, T, dk, dv, 64, kda.KDA_BF16, kda.KDA_BF16, 0)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = kda.library().kda_chunk_fwd_noalloc(ctypes.byref(desc), P(q), P(k), P(v), P(la), P(beta), P(S0), P(o),
                                             P(S_T), ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    assert st == 0, kda.library().kda_status_string(st).decode()
    return o, S_T


@pytest.mark.parametrize("shapes", [((1, 8, 64 * 40 + 17, 128), (1, 3, 200, 128)),
                                    ((2, 6, 64 * 23 + 5, 64), (1, 2, 70, 64))])
def test_noalloc_matches_allocating_call(shapes):
    for i, (B, H, T, d) in enumerate(shapes):
        say("noalloc call %d: B=%d H=%d T=%d d=%d" % (i, B, H, T, d))
        q, k, v, la, beta, S0 = synth.prefill_inputs(B, H, T, d, d, BF16, device=DEV, seed_base=9500 + 100 * i + d,
                                                     s0_std=0.3)
        need = kda.chunk_workspace_bytes(q, v)
        assert 0 < need <= kda.SCRATCH_BYTES
        o1, S1 = noalloc_call(q, k, v, la, beta, S0)
        o2, S2 = kda.chunk_fwd(q, k, v, la, beta, S0)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(S1, S2)
        o_ref, S_ref = oracle_prefill(q, k, v, la, beta, S0)
        eo = max_abs(host32(o1).reshape(B * H, T, d), o_ref)
        es = rel_l2_per_lane(host32(S1).reshape(B * H, d, d), S_ref)
        say("noalloc call %d: identical to kda_chunk_fwd; max|o-o_ref| %.3e relL2(S) %.3e" % (i, eo, es))
        assert eo <= TOL_O[BF16] and es <= TOL_S[BF16]
