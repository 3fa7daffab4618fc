"""GPU parity of kda_chunk_bwd (backward of chunkwise prefill) against the fp64 reverse-mode
oracle (oracle/backward.py, pinned to finite differences and autograd).

Tolerance: the backward differentiates around the forward's recomputed states, so its error
follows theirs; every gradient tensor is held per lane to the state bar, rel-L2 <= 1e-2, and to
max-abs <= 2e-2 of the lane's largest reference entry."""
import numpy as np
import pytest
import torch

import gated_delta_rule_78_amd as kda
from gated_delta_rule_78_amd import synth
from oracle import backward
from tests.parity import host32, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
BF16, F32 = torch.bfloat16, torch.float32


def check_grads(tag, got, ref, lanes):
    names = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")
    worst = []
    for name, g, r in zip(names, got, ref):
        g = host32(g).reshape(lanes, -1).astype(np.float64)
        r = np.asarray(r, np.float64).reshape(lanes, -1)
        num = np.linalg.norm(g - r, axis=1)
        den = np.maximum(np.linalg.norm(r, axis=1), 1e-300)
        rl2 = float(np.max(num / den))
        mx = float(np.max(np.max(np.abs(g - r), axis=1) / np.maximum(np.max(np.abs(r), axis=1), 1e-300)))
        worst.append("%s relL2 %.2e maxrel %.2e" % (name, rl2, mx))
        assert rl2 <= 1e-2 and mx <= 2e-2, "%s: %s rel-L2 %.3e, max-abs/max %.3e" % (tag, name, rl2, mx)
    say("%s: %s" % (tag, "; ".join(worst)))


def run_bwd(tag, B, H, T, dk, dv, odt=BF16, s0=True, dst=True, seed=7000, la_range=synth.LOG_ALPHA_RANGE):
    say("%s: B=%d H=%d T=%d dk=%d dv=%d dO=%s S0=%s dS_T=%s log_alpha=%s" % (tag, B, H, T, dk, dv, odt, s0, dst, la_range))
    q, k, v, la, beta, S0 = synth.prefill_inputs(B, H, T, dk, dv, BF16, device=DEV, seed_base=seed,
                                                 s0_std=0.3 if s0 else None, log_alpha_range=la_range)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 1)
    dO = torch.randn(B, H, T, dv, generator=g, device=DEV).to(odt)
    dST = torch.randn(B, H, dk, dv, generator=g, device=DEV) * 0.1 if dst else None
    got = kda.chunk_bwd(q, k, v, la, beta, S0, dO, dST)
    torch.cuda.synchronize()
    L = B * H
    f = lambda x: None if x is None else host32(x).reshape((L,) + tuple(x.shape[2:]))
    ref = backward.kda_bwd(f(q), f(k), f(v), f(la), f(beta), f(S0), f(dO), f(dST))
    check_grads(tag, got, ref, L)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_bwd_lengths(T):
    run_bwd("bwd T=%d" % T, 1, 2, T, 128, 128, seed=7000 + T)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_bwd_shapes_fp32_dO(dk, dv):
    run_bwd("bwd shapes", 2, 1, 150, dk, dv, odt=F32, seed=7100 + dk + dv)


def test_bwd_no_prefix_state_no_state_grad():
    run_bwd("bwd zero S0 / dS_T", 1, 2, 130, 128, 128, s0=False, dst=False, seed=7200)


def test_bwd_full_decay_domain():
    run_bwd("bwd full decay", 1, 2, 192, 128, 128, la_range=(-5.0, 0.0), seed=7300)


def test_bwd_strongest_decay_everywhere():
    """log_alpha = -5 on every channel and step (the contract's bound): inside a diagonal 16-token
    block the prep kernel's split decay factors then reach e^-75 and e^75."""
    run_bwd("bwd log_alpha = -5", 1, 2, 192, 128, 128, la_range=(-5.0, -5.0), seed=7350)


def test_bwd_many_lanes():
    """64 lanes: the reverse state pass takes blocks of 32 value columns here (it narrows them to
    16 when there are too few lanes to fill the GPU, as in the other cases)."""
    run_bwd("bwd 64 lanes", 2, 32, 130, 128, 128, seed=7500)


def test_bwd_full_workload_sampled_lanes():
    """The 8K workload in the configuration the benchmark times (B=1, H=32, T=8192, d=128, bf16,
    library plan, dS_T given): every gradient of heads 0 and 31 against the oracle, one lane at a
    time (the oracle keeps all 8192 states of a lane)."""
    w = synth.PREFILL_BF16_8K
    say("bwd 8K: %s, heads 0 and 31 against the oracle" % w.name)
    q, k, v, la, beta, S0 = synth.workload_inputs(w, device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(17)
    dO = torch.randn(w.B, w.H, w.T, w.d, generator=g, device=DEV).to(BF16)
    dST = torch.randn(w.B, w.H, w.d, w.d, generator=g, device=DEV) * 0.1
    got = kda.chunk_bwd(q, k, v, la, beta, S0, dO, dST)
    torch.cuda.synchronize()
    for h in (0, w.H - 1):
        f = lambda x: None if x is None else host32(x[:, h:h + 1]).reshape((1,) + tuple(x.shape[2:]))
        ref = backward.kda_bwd(f(q), f(k), f(v), f(la), f(beta), f(S0), f(dO), f(dST))
        check_grads("bwd 8K head %d" % h, [x[:, h:h + 1] for x in got], ref, 1)


def test_bwd_full_launch_slow_decay():
    """The 8K launch (B=1, H=32, T=8192) under slow decay, log_alpha ~ U[-0.02, 0], with S0 and
    dS_T: the state gradient carried back through all 128 chunks stays significant (under the
    workload's decay it fades within a few chunks). Head 13 against the oracle."""
    w = synth.PREFILL_BF16_8K
    say("bwd 8K slow decay: head 13 against the oracle")
    q, k, v, la, beta, S0 = synth.prefill_inputs(w.B, w.H, w.T, w.d, w.d, BF16, device=DEV, seed_base=7600,
                                                 s0_std=0.3, log_alpha_range=(-0.02, 0.0))
    g = torch.Generator(device=DEV)
    g.manual_seed(7601)
    dO = torch.randn(w.B, w.H, w.T, w.d, generator=g, device=DEV).to(BF16)
    dST = torch.randn(w.B, w.H, w.d, w.d, generator=g, device=DEV) * 0.1
    got = kda.chunk_bwd(q, k, v, la, beta, S0, dO, dST)
    torch.cuda.synchronize()
    h = 13
    f = lambda x: None if x is None else host32(x[:, h:h + 1]).reshape((1,) + tuple(x.shape[2:]))
    ref = backward.kda_bwd(f(q), f(k), f(v), f(la), f(beta), f(S0), f(dO), f(dST))
    check_grads("bwd 8K slow decay head %d" % h, [x[:, h:h + 1] for x in got], ref, 1)


def test_bwd_longer_sequence():
    """1024 tokens (16 chunks; the forward recompute splits the sequence into segments)."""
    run_bwd("bwd 1K", 1, 4, 1024, 128, 128, seed=7400)


def test_bwd_empty_sequence():
    q, k, v, la, beta, S0 = synth.prefill_inputs(1, 2, 0, 128, 128, BF16, device=DEV, s0_std=0.3)
    dST = torch.randn(1, 2, 128, 128, device=DEV)
    dO = torch.empty(1, 2, 0, 128, device=DEV, dtype=BF16)
    dq, dk, dv, dla, db, dS0 = kda.chunk_bwd(q, k, v, la, beta, S0, dO, dST)
    torch.cuda.synchronize()
    assert torch.equal(dS0, dST) and dq.numel() == 0


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_bwd_run_to_run_bitwise(dk, dv):
    """Every reduction of the backward runs in a fixed order (no float atomics): two calls on the
    same inputs give the same gradients bit for bit, across several chunks and lanes."""
    B, H, T = 1, 6, 64 * 9 + 13
    say("bwd determinism: B=%d H=%d T=%d dk=%d dv=%d" % (B, H, T, dk, dv))
    q, k, v, la, beta, S0 = synth.prefill_inputs(B, H, T, dk, dv, BF16, device=DEV, seed_base=7900 + dk,
                                                 s0_std=0.3)
    g = torch.Generator(device=DEV)
    g.manual_seed(7901)
    dO = torch.randn(B, H, T, dv, generator=g, device=DEV).to(BF16)
    dST = torch.randn(B, H, dk, dv, generator=g, device=DEV) * 0.1
    a = kda.chunk_bwd(q, k, v, la, beta, S0, dO, dST)
    b = kda.chunk_bwd(q, k, v, la, beta, S0, dO, dST)
    torch.cuda.synchronize()
    for name, x, y in zip(("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0"), a, b):
        assert torch.equal(x, y), name
