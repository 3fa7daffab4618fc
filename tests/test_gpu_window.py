"""GPU parity of the window split of the state pass. Each segment boundary first runs the last 8
chunks before it from a zero state (the affine pair of section 2.5 of the Kimi K3 reading notes
over that window). Where the window's transition M is exactly zero in fp32, its S~ is the exact
state at the boundary, and the lane runs every segment at once from those states. Elsewhere the
lane takes the full affine-pair split with the segment scan. Both paths, their mix in one launch,
windows that reach the lane's first chunk (and so S0), and packed batches whose short sequences
leave segments empty are checked against the fp64 oracle. The workspace's window flags (documented
in include/kda.h) show which path each lane took."""
import numpy as np
import pytest
import torch

import gated_delta_rule_78_amd as kda
from gated_delta_rule_78_amd import synth
from tests.parity import assert_close, host32, oracle_prefill, say
from tests.test_gpu_varlen import run_packed

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
BF16 = torch.bfloat16
SLOW = (-0.02, 0.0)


TWO = kda.STATE_PASS_TWO_KERNELS


def window_flags(ws, need, lanes, T, segments):
    """Flags [lanes, nseg - 1] of a fixed-length two-kernel call with a forced segment count: the
    workspace's last lanes * nseg int32 (no slot table in a fixed-length call)."""
    nchunks = (T + 63) // 64
    cps = (nchunks + segments - 1) // segments
    nseg = (nchunks + cps - 1) // cps
    f = ws[need - lanes * nseg * 4:need].view(torch.int32).view(lanes, nseg)
    return f[:, :nseg - 1].cpu().numpy()


def run_with_flags(tag, q, k, v, la, beta, S0, segments):
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    need = kda.chunk_workspace_bytes(q, v, segments=segments, state_pass=TWO)
    ws = torch.empty(need, device=DEV, dtype=torch.uint8)
    o, S_T = kda.chunk_fwd(q, k, v, la, beta, S0, segments=segments, state_pass=TWO, workspace=ws)
    torch.cuda.synchronize()
    flags = window_flags(ws, need, B * H, T, segments)
    say("%s: window flags per lane %s" % (tag, flags.tolist()))
    o_ref, S_ref = oracle_prefill(q, k, v, la, beta, S0)
    assert_close(tag, BF16, host32(o).reshape(B * H, T, dv), o_ref, host32(S_T).reshape(B * H, dk, dv), S_ref)
    return flags


def test_window_split_mixed_lanes():
    """Heads 0 and 2 at the workload decay take the window path; heads 1 and 3 at slow decay fall
    back to the affine-pair split, in the same launches (41 chunks in 4 segments of 11)."""
    B, H, T, d = 1, 4, 64 * 40 + 17, 128
    say("window mixed lanes: B=%d H=%d T=%d" % (B, H, T))
    q, k, v, la, beta, S0 = synth.prefill_inputs(B, H, T, d, d, BF16, device=DEV, seed_base=8000, s0_std=0.3)
    la_slow = synth.prefill_inputs(B, H, T, d, d, BF16, device=DEV, seed_base=8100, log_alpha_range=SLOW)[3]
    la[:, 1::2] = la_slow[:, 1::2]
    flags = run_with_flags("window mixed", q, k, v, la, beta, S0, segments=4)
    assert (flags[0::2] == 1).all() and (flags[1::2] == 0).all()


@pytest.mark.parametrize("decay", ["workload", "slow"])
def test_window_from_first_chunk_with_S0(decay):
    """Segments of 4 chunks: the windows before boundaries 1 and 2 reach back to chunk 0 and start
    from S0, so they are exact whatever the decay. The window before boundary 3 covers chunks 4..11:
    exact at the workload decay (every lane on the window path), not at slow decay (fallback)."""
    B, H, T, d = 1, 3, 64 * 12 + 5, 128
    la_range = synth.LOG_ALPHA_RANGE if decay == "workload" else SLOW
    say("window from chunk 0: B=%d H=%d T=%d decay=%s" % (B, H, T, decay))
    q, k, v, la, beta, S0 = synth.prefill_inputs(B, H, T, d, d, BF16, device=DEV, seed_base=8200, s0_std=0.5,
                                                 log_alpha_range=la_range)
    flags = run_with_flags("window chunk 0 " + decay, q, k, v, la, beta, S0, segments=4)
    assert (flags[:, :2] == 1).all()
    assert (flags[:, 2] == (1 if decay == "workload" else 0)).all()


def test_window_split_packed_empty_segments():
    """A packed batch split in 5 segments at the workload decay: the windows of segments past a
    short sequence's end cover that sequence's last chunks (or all of them, from S0), so every
    lane takes the window path, empty sequence included."""
    run_packed("window packed", [1500, 200, 0, 64 * 9 + 5, 3000], 4, 128, 128, 512, segments=5, seed=8300)


def test_window_split_dk64_dv128_fp32_out():
    """The window role at dk = 64, dv = 128 (M columns in other waves than at d = 128), fp32 output."""
    B, H, T = 2, 2, 64 * 30 + 3
    say("window dk64 dv128: B=%d H=%d T=%d" % (B, H, T))
    q, k, v, la, beta, S0 = synth.prefill_inputs(B, H, T, 64, 128, BF16, device=DEV, seed_base=8400, s0_std=0.3)
    need = kda.chunk_workspace_bytes(q, v, segments=3)
    ws = torch.empty(need, device=DEV, dtype=torch.uint8)
    o, S_T = kda.chunk_fwd(q, k, v, la, beta, S0, out_dtype=torch.float32, segments=3, workspace=ws)
    torch.cuda.synchronize()
    flags = window_flags(ws, need, B * H, T, 3)
    o_ref, S_ref = oracle_prefill(q, k, v, la, beta, S0)
    assert_close("window dk64", BF16, host32(o).reshape(B * H, T, 128), o_ref, host32(S_T).reshape(B * H, 64, 128),
                 S_ref)
    assert (flags == 1).all(), flags


def _random_cases(n, seed):
    """Seeded fixed-length cases around the split's edges: T near multiples of 64 and of the window,
    forced segment counts up to past the chunk count, decay per head from three ranges."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dk, dv = [(128, 128), (64, 128), (128, 64), (64, 64)][int(rng.integers(0, 4))]
        nch = int(rng.integers(1, 41))
        T = max(1, 64 * nch - int(rng.choice([0, 0, 1, 17, 63])))
        seg = int(rng.choice([0, 2, 3, 4, 5, 7, 9, 16, 64]))
        cases.append((i, int(rng.integers(1, 3)), int(rng.integers(1, 4)), T, dk, dv, seg,
                      bool(rng.integers(0, 2)), [int(x) for x in rng.integers(0, 3, 3)]))
    return cases


@pytest.mark.parametrize("case", _random_cases(24, 8500), ids=lambda c: "c%d" % c[0])
def test_split_random_shapes(case):
    """24 seeded shapes: every lane against the oracle, with each head's decay drawn from the
    workload range, slow decay or the full domain, so that window, fallback and mixed launches all
    occur at ragged lengths and forced segment counts."""
    i, B, H, T, dk, dv, seg, s0, kinds = case
    ranges = [synth.LOG_ALPHA_RANGE, SLOW, (-5.0, 0.0)]
    say("random split %d: B=%d H=%d T=%d dk=%d dv=%d segments=%d S0=%s decay kinds %s" % (i, B, H, T, dk, dv, seg, s0, kinds[:H]))
    q, k, v, la, beta, S0 = synth.prefill_inputs(B, H, T, dk, dv, BF16, device=DEV, seed_base=8600 + 10 * i,
                                                 s0_std=0.3 if s0 else None)
    for h in range(H):
        lr = ranges[kinds[h]]
        la[:, h] = synth.prefill_inputs(B, H, T, dk, dv, BF16, device=DEV, seed_base=8700 + 10 * i + h,
                                        log_alpha_range=lr)[3][:, h]
    o, S_T = kda.chunk_fwd(q, k, v, la, beta, S0, segments=seg)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(q, k, v, la, beta, S0)
    assert_close("random split %d" % i, BF16, host32(o).reshape(B * H, T, dv), o_ref,
                 host32(S_T).reshape(B * H, dk, dv), S_ref)


@pytest.mark.parametrize("order", ["fast_then_slow", "slow_then_fast"])
def test_window_split_decay_changes_along_the_sequence(order):
    """One lane's decay changes halfway (41 chunks in 4 segments of 11): some of its windows are
    exact and some not. Fast then slow: segment 1 finishes from its window in the first launch and
    the fallback's pass 1 computes its affine pair for the scan; slow then fast: the middle
    segments compute their pairs in the first launch and the last segment finishes from its window."""
    B, H, T, d = 1, 2, 64 * 40 + 17, 128
    say("window decay change %s: B=%d H=%d T=%d" % (order, B, H, T))
    q, k, v, la, beta, S0 = synth.prefill_inputs(B, H, T, d, d, BF16, device=DEV, seed_base=8900, s0_std=0.3)
    la_slow = synth.prefill_inputs(B, H, T, d, d, BF16, device=DEV, seed_base=8950, log_alpha_range=SLOW)[3]
    half = 64 * 20
    if order == "fast_then_slow":
        la[:, :, half:] = la_slow[:, :, half:]
    else:
        la[:, :, :half] = la_slow[:, :, :half]
    flags = run_with_flags("window decay change " + order, q, k, v, la, beta, S0, segments=4)
    expect = [1, 0, 0] if order == "fast_then_slow" else [0, 0, 1]
    assert (flags == np.array(expect)).all(), flags


def _random_packed(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        N = int(rng.integers(1, 7))
        lens = [int(x) for x in rng.choice([0, 1, 63, 64, 65, 300, 700, 1300, 2100], N)]
        out.append((i, lens, int(rng.integers(1, 4)), int(rng.choice([0, 2, 3, 5, 9])), int(rng.choice([0, 64, 512])),
                    int(rng.integers(0, 3))))
    return out


@pytest.mark.parametrize("case", _random_packed(10, 9100), ids=lambda c: "p%d" % c[0])
def test_split_random_packed(case):
    """10 seeded packed batches (lengths from empty to 33 chunks, 1-6 sequences, forced or planned
    segment counts, checkpoints off, every 64 or every 512 tokens, one decay range per case): every
    lane, final state and checkpoint against the oracle."""
    i, lens, H, seg, E, kind = case
    la_range = [synth.LOG_ALPHA_RANGE, SLOW, (-5.0, 0.0)][kind]
    run_packed("random packed %d" % i, lens, H, 128, 128, E, segments=seg, seed=9200 + 10 * i, la_range=la_range)
