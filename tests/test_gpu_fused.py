"""GPU parity of the fused prefill (kda_chunk_desc::state_pass = 2): one kernel builds every chunk's
factors in LDS and runs the state step on them (section 2.2 chunk equations of the Kimi K3 reading
notes), its segments starting from the window states of section 2.5's sequence split, and lanes
with an inexact window falling back to the two-kernel path within the same call; with state
checkpoints and the fused gating through kda_chunk_fwd_varlen (equal lengths). Each case is
checked against the fp64 oracle; where the two paths split a lane the same way, the fused output
must also equal the two-kernel output bit for bit (the same per-chunk arithmetic in the same
order: only where the factors live differs)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_78_amd as kda
from gated_delta_rule_78_amd import synth
from oracle import gating, native
from tests.parity import TOL_S, assert_close, host32, oracle_prefill, rel_l2_per_lane, say
from tests.test_gpu_gating import EPS, G_MIN, check_gated

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
BF16 = torch.bfloat16
FUSED, TWO = kda.STATE_PASS_FUSED, kda.STATE_PASS_TWO_KERNELS
SLOW = (-0.02, 0.0)


def inputs(B, H, T, seed, s0_std=0.3, la_range=synth.LOG_ALPHA_RANGE):
    return synth.prefill_inputs(B, H, T, 128, 128, BF16, device=DEV, seed_base=seed, s0_std=s0_std,
                                log_alpha_range=la_range)


def check(tag, q, k, v, la, beta, S0, segments, out_dtype=None, same_as_two=True):
    B, H, T, _ = q.shape
    o, S_T = kda.chunk_fwd(q, k, v, la, beta, S0, out_dtype=out_dtype, segments=segments, state_pass=FUSED)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_prefill(q, k, v, la, beta, S0)
    assert_close(tag, BF16, host32(o).reshape(B * H, T, 128), o_ref, host32(S_T).reshape(B * H, 128, 128), S_ref)
    if same_as_two:
        o2, S2 = kda.chunk_fwd(q, k, v, la, beta, S0, out_dtype=out_dtype, segments=segments, state_pass=TWO)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(S_T, S2), "%s: fused and two-kernel outputs differ" % tag
        say("%s: bit-identical to the two-kernel path" % tag)
    return o, S_T


@pytest.mark.parametrize("T", [1, 63, 64, 65, 64 * 9 + 37])
def test_fused_one_segment_ragged(T):
    """One segment per lane (the fused kernel alone, no windows): ragged lengths, a prefix state."""
    say("fused one segment: B=2 H=3 T=%d" % T)
    q, k, v, la, beta, S0 = inputs(2, 3, T, 9400 + T)
    check("fused T=%d" % T, q, k, v, la, beta, S0, segments=1)


def test_fused_fp32_output_zero_state():
    say("fused fp32 out: B=1 H=2 T=1000 S0=None")
    q, k, v, la, beta, _ = inputs(1, 2, 1000, 9450, s0_std=None)
    check("fused fp32 out", q, k, v, la, beta, None, segments=3, out_dtype=torch.float32)


@pytest.mark.parametrize("segments", [2, 4, 7])
def test_fused_segments_from_windows(segments):
    """Forced splits at the workload decay: every window is exact, so every lane is fused."""
    T = 64 * 40 + 17
    say("fused segments=%d: B=1 H=4 T=%d" % (segments, T))
    q, k, v, la, beta, S0 = inputs(1, 4, T, 9500 + segments)
    check("fused segments=%d" % segments, q, k, v, la, beta, S0, segments=segments)


def test_fused_short_segments():
    """Segments of 2 chunks, shorter than the 8-chunk window: the windows reach back over several
    segments (and to chunk 0 and S0)."""
    T = 64 * 12 + 5
    say("fused short segments: B=1 H=2 T=%d segments=6" % T)
    q, k, v, la, beta, S0 = inputs(1, 2, T, 9550)
    check("fused short segments", q, k, v, la, beta, S0, segments=6)


def test_fused_slow_decay_falls_back():
    """Slow decay: no window is exact, every lane takes the two-kernel fallback inside the call."""
    T = 64 * 30 + 9
    say("fused slow decay: B=1 H=3 T=%d segments=4" % T)
    q, k, v, la, beta, S0 = inputs(1, 3, T, 9600, la_range=SLOW)
    check("fused slow decay", q, k, v, la, beta, S0, segments=4)


def test_fused_mixed_lanes():
    """Heads 1 and 3 at slow decay fall back; heads 0 and 2 are fused, in the same call."""
    T = 64 * 40 + 17
    say("fused mixed lanes: B=1 H=4 T=%d segments=4" % T)
    q, k, v, la, beta, S0 = inputs(1, 4, T, 9650)
    la_slow = inputs(1, 4, T, 9660, la_range=SLOW)[3]
    la[:, 1::2] = la_slow[:, 1::2]
    check("fused mixed lanes", q, k, v, la, beta, S0, segments=4)


@pytest.mark.parametrize("order", ["fast_then_slow", "slow_then_fast"])
def test_fused_decay_changes_along_the_sequence(order):
    """A lane with some exact windows and some inexact ones falls back as a whole."""
    T = 64 * 40 + 17
    say("fused decay change %s: B=1 H=2 T=%d" % (order, T))
    q, k, v, la, beta, S0 = inputs(1, 2, T, 9700)
    la_slow = inputs(1, 2, T, 9710, la_range=SLOW)[3]
    half = 64 * 20
    if order == "fast_then_slow":
        la[:, :, half:] = la_slow[:, :, half:]
    else:
        la[:, :, :half] = la_slow[:, :, :half]
    check("fused decay change " + order, q, k, v, la, beta, S0, segments=4)


def test_fused_in_place_state():
    """S_T written over S0 (the last segment writes it; every reader of S0 comes first)."""
    T = 64 * 20 + 3
    say("fused in place: B=2 H=2 T=%d segments=3" % T)
    q, k, v, la, beta, S0 = inputs(2, 2, T, 9750)
    o_ref, S_ref = oracle_prefill(q, k, v, la, beta, S0)
    S = S0.clone()
    o, S_T = kda.chunk_fwd(q, k, v, la, beta, S, segments=3, state_pass=FUSED, S_T=S)
    torch.cuda.synchronize()
    assert S_T.data_ptr() == S.data_ptr()
    assert_close("fused in place", BF16, host32(o).reshape(4, T, 128), o_ref, host32(S).reshape(4, 128, 128), S_ref)


def _random_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        nch = int(rng.integers(1, 49))
        T = max(1, 64 * nch - int(rng.choice([0, 0, 1, 31, 63])))
        out.append((i, int(rng.integers(1, 3)), int(rng.integers(1, 4)), T, int(rng.choice([0, 1, 2, 3, 5, 8, 16])),
                    bool(rng.integers(0, 2)), [int(x) for x in rng.integers(0, 3, 3)]))
    return out


@pytest.mark.parametrize("case", _random_cases(16, 9800), ids=lambda c: "f%d" % c[0])
def test_fused_random_shapes(case):
    """16 seeded shapes: ragged T up to 48 chunks, forced or planned segment counts, each head's
    decay from the workload range, slow decay or the full domain (fused, fallback and mixed)."""
    i, B, H, T, seg, s0, kinds = case
    say("fused random %d: B=%d H=%d T=%d segments=%d S0=%s decay kinds %s" % (i, B, H, T, seg, s0, kinds[:H]))
    q, k, v, la, beta, S0 = inputs(B, H, T, 9900 + 10 * i, s0_std=0.3 if s0 else None)
    ranges = [synth.LOG_ALPHA_RANGE, SLOW, (-5.0, 0.0)]
    for h in range(H):
        la[:, h] = inputs(B, H, T, 9905 + 10 * i + h, la_range=ranges[kinds[h]])[3][:, h]
    check("fused random %d" % i, q, k, v, la, beta, S0, segments=seg)


def test_fused_refused_for_dk64():
    q, k, v, la, beta, S0 = synth.prefill_inputs(1, 1, 128, 64, 128, BF16, device=DEV, seed_base=9990)
    with pytest.raises(kda.KDAError):
        kda.chunk_fwd(q, k, v, la, beta, S0, state_pass=FUSED)


def _equal_length_ckpt_ref(q, k, v, la, beta, S0, E):
    N, H, T, d = q.shape
    f = lambda t: host32(t).reshape((N * H,) + tuple(t.shape[2:]))
    o_ref, S_ref, ck_ref = native.kda_fwd(f(q), f(k), f(v), f(la), f(beta), None if S0 is None else f(S0), ckpt_every=E)
    n = T // E
    return o_ref, S_ref, ck_ref.reshape(N, H, n, d, d).transpose(0, 2, 1, 3, 4).reshape(N * n, H, d, d)


@pytest.mark.parametrize("E", [64, 512])
def test_fused_checkpoints_equal_lengths(E):
    """State checkpoints every E tokens (kda_chunk_fwd_varlen, equal lengths) from the fused kernel,
    one head at slow decay falling back: bit-identical to the two-kernel path, and against the
    oracle's prefix states."""
    N, H, T = 2, 3, 64 * 40 + 17
    say("fused checkpoints: N=%d H=%d T=%d E=%d segments=4" % (N, H, T, E))
    q, k, v, la, beta, S0 = inputs(N, H, T, 9600 + E)
    la[:, 2] = inputs(N, H, T, 9610 + E, la_range=SLOW)[3][:, 2]
    outs = {}
    for sp in (FUSED, TWO):
        outs[sp] = kda.chunk_fwd_varlen(q, k, v, la, beta, None, S0, ckpt_every=E, segments=4, state_pass=sp)
    torch.cuda.synchronize()
    for a, b in zip(outs[FUSED], outs[TWO]):
        assert torch.equal(a, b), "fused and two-kernel checkpoint calls differ"
    o, S_T, ck, offs = outs[FUSED]
    o_ref, S_ref, ck_ref = _equal_length_ckpt_ref(q, k, v, la, beta, S0, E)
    assert_close("fused checkpoints E=%d" % E, BF16, host32(o).reshape(N * H, T, 128), o_ref,
                 host32(S_T).reshape(N * H, 128, 128), S_ref)
    n = T // E
    assert np.array_equal(offs.cpu().numpy(), [s * n for s in range(N + 1)])
    es = rel_l2_per_lane(host32(ck[:N * n]).reshape(N * n * H, -1), ck_ref.reshape(N * n * H, -1))
    say("fused checkpoints E=%d: %d x %d states, relL2 = %.3e" % (E, N * n, H, es))
    assert es <= TOL_S[BF16]


@pytest.mark.parametrize("z_on,gate_on,odt", [(True, False, BF16), (False, True, BF16), (True, True, BF16),
                                               (True, True, torch.float32)])
def test_fused_gating_equal_lengths(z_on, gate_on, odt):
    """The fused decay prologue and gated RMSNorm epilogue in the fused kernel: bit-identical to
    the two-kernel path (which the gating tests hold to the oracle), and the gated output against
    the oracle's epilogue of the oracle's core output."""
    N, H, T, E = 1, 4, 64 * 24 + 5, 512
    say("fused gating: z=%s gate=%s out=%s N=%d H=%d T=%d" % (z_on, gate_on, odt, N, H, T))
    q, k, v, la, beta, S0 = inputs(N, H, T, 9700 + 2 * z_on + gate_on)
    z, A_log, gate, w = synth.gating_inputs((N, H, T), H, 128, 128, BF16, device=DEV, seed=9720 + 2 * z_on + gate_on)
    kw = dict(ckpt_every=E, segments=3, out_dtype=odt)
    if z_on:
        kw.update(z=z, A_log=A_log, g_min=G_MIN)
    if gate_on:
        kw.update(gate=gate, norm_weight=w, eps=EPS)
    outs = {sp: kda.chunk_fwd_varlen(q, k, v, None if z_on else la, beta, None, S0, state_pass=sp, **kw)
            for sp in (FUSED, TWO)}
    torch.cuda.synchronize()
    for a, b in zip(outs[FUSED], outs[TWO]):
        assert torch.equal(a, b), "fused and two-kernel gated calls differ"
    o, S_T = outs[FUSED][0], outs[FUSED][1]
    g = gating.log_decay(host32(z), host32(A_log)[None, :, None, None], G_MIN).astype(np.float32) if z_on else host32(la)
    f = lambda t: np.asarray(t).reshape((N * H,) + tuple(np.asarray(t).shape[2:]))
    o_ref, S_ref = native.kda_fwd(f(host32(q)), f(host32(k)), f(host32(v)), f(g), f(host32(beta)), f(host32(S0)))
    if gate_on:
        check_gated("fused gating", o.reshape(N * H, T, 128), o_ref, gate.reshape(N * H, T, 128), w, odt)
        es = rel_l2_per_lane(host32(S_T).reshape(N * H, -1), S_ref.reshape(N * H, -1))
        assert es <= TOL_S[BF16]
    else:
        assert_close("fused prologue", BF16, host32(o).reshape(N * H, T, 128), o_ref, host32(S_T).reshape(N * H, 128, 128),
                     S_ref)


@pytest.mark.parametrize("segments", [1, 2])
def test_fused_more_workgroups_than_compute_units(segments):
    """300 lanes (x segments) of workgroups, more than one per compute unit: several rounds."""
    B, H, T = 3, 100, 64 * 6 + 11
    say("fused many lanes: B=%d H=%d T=%d segments=%d" % (B, H, T, segments))
    q, k, v, la, beta, S0 = inputs(B, H, T, 9950 + segments)
    check("fused many lanes segments=%d" % segments, q, k, v, la, beta, S0, segments=segments)


def _packed_pair(tag, lens, H, E, segments, seed, slow_heads=(), max_len=None, s0_std=0.3, odt=BF16, **gkw):
    """One packed batch through the fused plan and the two-kernel plan with the same split: every
    output equal bit for bit; returns the inputs and the fused outputs."""
    say("%s: lens=%s H=%d E=%d segments=%d slow heads=%s max_len=%s" % (tag, list(lens), H, E, segments,
                                                                        list(slow_heads), max_len))
    q, k, v, la, beta, cu, S0 = synth.packed_inputs(lens, H, 128, 128, BF16, device=DEV, seed_base=seed,
                                                    s0_std=s0_std)
    for h in slow_heads:
        la[h] = synth.packed_inputs(lens, H, 128, 128, BF16, device=DEV, seed_base=seed + 50,
                                    log_alpha_range=SLOW)[3][h]
    outs = {sp: kda.chunk_fwd_varlen(q, k, v, la if "z" not in gkw else None, beta, cu, S0, max_len=max_len,
                                     ckpt_every=E, segments=segments, state_pass=sp, out_dtype=odt, **gkw)
            for sp in (FUSED, TWO)}
    torch.cuda.synchronize()
    _same_packed(tag, outs[FUSED], outs[TWO])
    return (q, k, v, la, beta, cu, S0), outs[FUSED]


def _same_packed(tag, a, b):
    """o, S_T and the checkpoint offsets equal bit for bit, and the checkpoints written (the first
    offsets[N] of the buffer: the rest of its capacity is never written)."""
    for x, y in zip(a[:2], b[:2]):
        assert torch.equal(x, y), "%s: fused and two-kernel packed calls differ" % tag
    if a[3] is not None:
        assert torch.equal(a[3], b[3]), "%s: checkpoint offsets differ" % tag
        n = int(a[3][-1])
        assert torch.equal(a[2][:n], b[2][:n]), "%s: checkpoints differ" % tag
    say("%s: bit-identical to the two-kernel path" % tag)


def _check_packed_oracle(tag, ins, outs, E, N, H):
    q, k, v, la, beta, cu, S0 = ins
    o, S_T, ck, offs = outs
    ref = native.kda_varlen(host32(q), host32(k), host32(v), host32(la), host32(beta), cu.cpu().numpy(),
                            None if S0 is None else host32(S0), ckpt_every=E)
    assert_close(tag, BF16, host32(o), ref[0], host32(S_T).reshape(N * H, 128, 128), ref[1].reshape(N * H, 128, 128))
    if E:
        assert np.array_equal(offs.cpu().numpy(), np.asarray(ref[3]))
        n = int(ref[3][-1])
        if n:
            es = rel_l2_per_lane(host32(ck[:n]).reshape(n * H, -1), ref[2].reshape(n * H, -1))
            say("%s: %d checkpoints x %d heads, relL2 = %.3e" % (tag, n, H, es))
            assert es <= TOL_S[BF16]


PACKED_MIXES = {
    "ragged": [1000, 64, 0, 1, 513, 700, 130, 77],
    "one_long": [40, 2600, 17],
    "boundaries": [64 * 12, 64 * 12 - 1, 64 * 12 + 1, 64 * 4, 64 * 8],
}


@pytest.mark.parametrize("segments", [1, 3, 5])
@pytest.mark.parametrize("mix", list(PACKED_MIXES))
def test_fused_packed_mixes(mix, segments):
    """Packed sequences of mixed lengths (empty, one token, chunk multiples, the longest well past
    the others) with checkpoints every 128 tokens: segments past a short sequence's end are empty,
    and its windows are clamped to its chunks."""
    lens, H, E = PACKED_MIXES[mix], 3, 128
    ins, outs = _packed_pair("fused packed %s" % mix, lens, H, E, segments, 12000 + 10 * segments + len(mix))
    _check_packed_oracle("fused packed %s segments=%d" % (mix, segments), ins, outs, E, len(lens), H)


def test_fused_packed_slow_heads_fall_back():
    """Slow decay on two of four heads: their lanes' windows are inexact, every record is then
    built and the two-kernel passes finish those lanes; the other lanes stay fused."""
    lens, H, E = [64 * 30 + 9, 300, 64 * 17], 4, 256
    ins, outs = _packed_pair("fused packed slow", lens, H, E, 4, 12500, slow_heads=(1, 3))
    _check_packed_oracle("fused packed slow", ins, outs, E, len(lens), H)


def test_fused_packed_max_len_and_empty():
    """max_len above the longest sequence (the plan's chunk count), and a batch of empty sequences."""
    lens, H = [700, 64 * 10, 5], 2
    ins, outs = _packed_pair("fused packed max_len", lens, H, 64, 3, 12600, max_len=64 * 16)
    _check_packed_oracle("fused packed max_len", ins, outs, 64, len(lens), H)
    ins, outs = _packed_pair("fused packed empty", [0, 0, 0], 2, 0, 2, 12700, s0_std=0.2)
    o, S_T = outs[0], outs[1]
    assert o.numel() == 0 and torch.equal(S_T, ins[6])


def test_fused_packed_many_short_sequences():
    """Sixty sequences of at most three chunks under a 3-segment plan of a longer one: most lanes
    have all their chunks in segment 0, and their windows start at chunk 0."""
    g = np.random.default_rng(12800)
    lens = [int(x) for x in g.integers(0, 64 * 3, 60)] + [64 * 20 + 3]
    ins, outs = _packed_pair("fused packed many", lens, 2, 64, 3, 12800, s0_std=None)
    _check_packed_oracle("fused packed many", ins, outs, 64, len(lens), 2)


@pytest.mark.parametrize("odt", [BF16, torch.float32])
def test_fused_packed_gating(odt):
    """The decay prologue and gated RMSNorm epilogue on a packed batch in the fused kernel:
    bit-identical to the two-kernel path; the gated output against the oracle's epilogue."""
    lens, H, E = [64 * 14 + 30, 0, 200, 64 * 9], 3, 256
    z_seed = 12900 + (odt == BF16)
    q, k, v, la, beta, cu, S0 = synth.packed_inputs(lens, H, 128, 128, BF16, device=DEV, seed_base=z_seed, s0_std=0.3)
    T = int(cu[-1])
    z, A_log, gate, w = synth.gating_inputs((H, T), H, 128, 128, BF16, device=DEV, seed=z_seed + 1)
    kw = dict(z=z, A_log=A_log, g_min=G_MIN, gate=gate, norm_weight=w, eps=EPS, ckpt_every=E, segments=3,
              out_dtype=odt)
    say("fused packed gating: lens=%s H=%d out=%s" % (lens, H, odt))
    outs = {sp: kda.chunk_fwd_varlen(q, k, v, None, beta, cu, S0, state_pass=sp, **kw) for sp in (FUSED, TWO)}
    torch.cuda.synchronize()
    _same_packed("fused packed gating", outs[FUSED], outs[TWO])
    o, S_T = outs[FUSED][0], outs[FUSED][1]
    g = gating.log_decay(host32(z), host32(A_log)[:, None, None], G_MIN).astype(np.float32)
    ref = native.kda_varlen(host32(q), host32(k), host32(v), g, host32(beta), cu.cpu().numpy(), host32(S0))
    check_gated("fused packed gating", o, ref[0], gate, w, odt)
    N = len(lens)
    es = rel_l2_per_lane(host32(S_T).reshape(N * H, -1), ref[1].reshape(N * H, -1))
    assert es <= TOL_S[BF16]


@pytest.mark.parametrize("segments", [2, 3])
def test_fused_packed_workload_sampled_heads(segments):
    """The packed 8K workload (12 sequences of 27 to 2500 tokens, 32 heads, checkpoints every 512)
    forced onto the fused path: bit-identical to the two-kernel path with the same split, and the
    oracle checks 3 heads of every sequence."""
    w = synth.PACKED_BF16_8K
    lens = synth.PACKED_BF16_8K_LENS
    say("fused packed workload: segments=%d" % segments)
    q, k, v, la, beta, cu, S0 = synth.packed_inputs(lens, w.H, w.d, w.d, BF16, device=DEV)
    outs = {sp: kda.chunk_fwd_varlen(q, k, v, la, beta, cu, None, max_len=max(lens), ckpt_every=512, segments=segments,
                                     state_pass=sp) for sp in (FUSED, TWO)}
    torch.cuda.synchronize()
    _same_packed("fused packed workload", outs[FUSED], outs[TWO])
    o, S_T, ck, offs = outs[FUSED]
    heads = [0, 13, 31]
    sub = lambda x: host32(x[heads])
    ref = native.kda_varlen(sub(q), sub(k), sub(v), sub(la), sub(beta), cu.cpu().numpy(), None, ckpt_every=512)
    N = len(lens)
    assert_close("fused packed workload (3 heads)", BF16, host32(o[heads]), ref[0],
                 host32(S_T[:, heads]).reshape(N * 3, w.d, w.d), ref[1].reshape(N * 3, w.d, w.d))
    assert np.array_equal(offs.cpu().numpy(), np.asarray(ref[3]))
    n = int(ref[3][-1])
    es = rel_l2_per_lane(host32(ck[:n][:, heads]).reshape(n * 3, -1), ref[2].reshape(n * 3, -1))
    say("fused packed workload: %d checkpoints x 3 heads, relL2 = %.3e" % (n, es))
    assert es <= TOL_S[BF16]
